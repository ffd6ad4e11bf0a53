/*
 * kvq.h -- C ABI of libkvq.so: Block-GTQ key-cache quantization and packed-cache
 * decode attention for AMD Instinct MI355X (gfx950).
 *
 * The method is the one on the page "RoPE-Aware Bit Allocation for KV-Cache
 * Quantization" (abstract): under RoPE a cached key's contribution to a later
 * logit splits into 2-D frequency blocks; per layer and KV head a label-free
 * energy is scored per block; integer bit widths are handed out greedily by
 * marginal gain on top of a TQ-MSE scalar quantizer; a packed cache is then read
 * by a decode-attention path.  The concrete numeric reading (per-token L2 norm,
 * per-block scale, Gaussian Lloyd-Max codebooks, packed layout v1) is fixed by the
 * comments below.
 *
 * Conventions for every call:
 *  - All buffers are owned by the caller; pointers marked "device" are device
 *    memory on the current HIP device.  The library allocates no device memory
 *    and keeps no pointer after returning (the one device buffer of its own is the
 *    fixed array of kvq_packed_decode_attn_noalloc, reserved when the library is
 *    loaded on a GPU).
 *  - `stream` is a hipStream_t (NULL = default stream).  Calls enqueue work and
 *    return without synchronising; asynchronous faults surface at the caller's
 *    next synchronisation.
 *  - Arguments are validated on the host BEFORE any HIP call; on failure nothing
 *    is launched or written and a negative kvq_status is returned.
 *  - Element strides are in elements (binary16), not bytes.
 *  - No call aborts, exits or throws.  Calls on different streams may run
 *    concurrently; calls that write the same buffer must be ordered by the caller.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_LAYOUT_VERSION 1
#define KVQ_TILE_TOKENS 64

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_ARG = -1,        /* null pointer, bad enum, n < 0 */
    KVQ_ERR_SHAPE = -2,      /* unsupported head_dim, n_kv_heads, GQA ratio */
    KVQ_ERR_BUDGET = -3,     /* budget outside [0, 8*d/2] and != 16*d/2; UNIFORM not divisible; v_bits invalid */
    KVQ_ERR_ALIGN = -4,      /* pointer or stride below the alignment a call requires */
    KVQ_ERR_CAPACITY = -5,   /* capacity not a multiple of 64, or max_len/max_new beyond it */
    KVQ_ERR_WORKSPACE = -6,  /* workspace too small */
    KVQ_ERR_HIP = -7,        /* a HIP launch failed */
    KVQ_ERR_VERSION = -8     /* layout_version != KVQ_LAYOUT_VERSION */
} kvq_status;

/* RoPE block map (which two coordinates form 2-D frequency block i) */
#define KVQ_PAIR_HALF 0          /* block i = (i, i + d/2): rotate-half convention (default) */
#define KVQ_PAIR_INTERLEAVED 1   /* block i = (2i, 2i + 1) */

/* allocation modes */
#define KVQ_GREEDY 0             /* Block-GTQ greedy marginal-gain allocation */
#define KVQ_UNIFORM 1            /* every block budget/(d/2) bits (values, uniform baseline) */

/* decode kernel choice for kvq_packed_decode_attn_ex */
#define KVQ_DECODE_AUTO 0
#define KVQ_DECODE_GENERIC 1     /* any widths incl. 16-bit passthrough, GQA ratio <= 16 */
#define KVQ_DECODE_MFMA 2        /* K widths 0..8 (budget <= 256), v_bits 1..8 or 16, GQA ratio <= 8 */

typedef struct {
    int32_t layout_version;  /* KVQ_LAYOUT_VERSION */
    int32_t head_dim;        /* d: 128 for quantize/attention; even, 2..128 for energy/allocation */
    int32_t n_kv_heads;      /* KV heads of one layer, >= 1 */
    int32_t rope_pairing;    /* KVQ_PAIR_HALF or KVQ_PAIR_INTERLEAVED */
    int32_t k_budget;        /* sum of the d/2 key block widths: 0..8*(d/2), or exactly 16*(d/2) (passthrough) */
    int32_t v_bits;          /* uniform value width: 1..8, or 16 (passthrough) */
    int64_t capacity_tokens; /* token slots per sequence and layer; multiple of 64 */
} kvq_geom;

/* Packed layout v1 (per sequence and layer):  [n_kv_heads][capacity/64 tiles][tile].
 * Tile of 64 token slots:
 *   K section: 64 records of SK = 16*ceil(2*k_budget/128) bytes.  Record p holds slot
 *              p's key codes as an LSB-first bitstream (bit b of the stream is bit
 *              b%8 of byte b/8) in "K order": blocks sorted by width descending
 *              (ties: lower block index first), each block contributing coordinate
 *              p(i) then q(i), width-0 blocks omitted; a field is w bits (16 bits =
 *              raw binary16 for passthrough).
 *   V section: d runs of 8*v_bits bytes; run c holds slot p's value code of
 *              coordinate c at bits [p*v_bits, (p+1)*v_bits).
 *   64 binary32 key scales, then 64 binary32 value scales (per-token L2 norms).
 * Unused slots are zero; the cache must be zero-initialised before first use. */

int32_t kvq_version(void);                        /* KVQ_LAYOUT_VERSION */
const char *kvq_status_string(int32_t status);    /* static string, never NULL */

/* Bytes of one tile, of one sequence's region for one layer, or a negative
 * kvq_status if the geometry is invalid. */
int64_t kvq_tile_bytes(const kvq_geom *g);
int64_t kvq_cache_bytes(const kvq_geom *g);

/* Host copy of the built-in codebook for width w (1..8): 2^w binary16 levels
 * (ascending), 2^w binary32 thresholds (entry 0 unused; entry j is the midpoint of
 * levels j-1 and j), and the 8 binary32 distortion drops dD[b] = D(b) - D(b+1) of
 * Gaussian Lloyd-Max quantization (D(0) = 1) used as greedy gains.  Any output
 * pointer may be NULL.  No GPU access. */
int32_t kvq_get_codebook(int32_t w, uint16_t *levels_fp16, float *thresholds, float *gain_dd);

/* a1 -- Block energy.  The page ("RoPE-Aware Bit Allocation...", abstract) scores
 * each RoPE block of each KV head with a label-free energy.  Reading: the exact sum
 * over the given tokens of k_{p(i)}^2 + k_{q(i)}^2.  Every binary16 square is a
 * multiple of 2^-48, so the sum is kept exactly as an unsigned 128-bit count of
 * 2^-48 units; results are independent of order, tiling and launch shape.
 *   x       : device binary16, element (t, h, c) at x[t*stride_tok + h*stride_head + c],
 *             t < n_tok, h < n_kv_heads, c < head_dim (c contiguous)
 *   energy  : device uint64 [n_kv_heads][head_dim/2][2] = (low, high) limbs;
 *             ACCUMULATED INTO (zero it for a fresh sum; call repeatedly to add tokens)
 * Requirements: head_dim even, 2..128; n_tok >= 0; x 4-byte aligned with even
 * strides; energy 16-byte aligned.  The whole geometry must be valid. */
int32_t kvq_block_energy(const kvq_geom *g, const void *x, int64_t n_tok, int64_t stride_tok,
                         int64_t stride_head, uint64_t *energy, void *stream);

/* a2 -- Bit allocation (page abstract: greedy integer widths by marginal gain under
 * a fixed budget, per layer and KV head).  Per unit (row of `energy`):
 *   E_i = RN64(energy_i * 2^-48) (correctly rounded from the exact integer);
 *   GREEDY: from b = 0, `budget` times give one bit to the block maximising
 *           RN64(E_i * dD[b_i]) among blocks with b_i < 8; ties -> lowest index;
 *   UNIFORM: b_i = budget/(d/2) (budget must be divisible);
 *   budget == 16*(d/2): every block 16 (raw passthrough), either mode;
 *   sigma_i = RN32(sqrt(E_i / (2*E_tot))), E_tot = RN64(sum_i energy_i * 2^-48); 0 if E_tot = 0.
 *   energy : device uint64 [n_units][head_dim/2][2]
 *   bits   : device uint8  [n_units][head_dim/2]
 *   sigma  : device float  [n_units][head_dim/2]
 * The call uses g->head_dim (the whole geometry must be valid).  Requirements:
 * budget in [0, 8*(d/2)] or == 16*(d/2); energy 16-byte aligned. */
int32_t kvq_allocate_bits(const kvq_geom *g, const uint64_t *energy, int32_t n_units, int32_t budget,
                          int32_t mode, uint8_t *bits, float *sigma, void *stream);

/* a3 -- Quantize and pack (page abstract: TQ-MSE codes at the allocated widths,
 * stored in a packed cache).  For sequence s (< n_seq) the n_new[s] token rows
 * src_row0[s] .. src_row0[s]+n_new[s]-1 of k and v are written to slots
 * first_slot[s] .. of the region cache + seq_byte_off[s].  Per token and head:
 *   s_t = sqrtf(pairwise binary32 tree of the squared coordinates, coordinate order);
 *   code_c = #{ j in 1..2^w-1 : x_c >= RN32(s_t * RN32(sigma_i * thr_w[j])) } for
 *            width w = 1..8 (w = 16: raw binary16 bits; w = 0: nothing stored).
 * Keys use k_bits/k_sigma; values use width v_bits and v_sigma.
 *   k, v        : device binary16 rows, element (r, h, c) at base[r*stride_tok + h*stride_head + c]
 *   first_slot, src_row0, seq_byte_off : device int64 [n_seq];  n_new : device int32 [n_seq]
 *   k_bits      : device uint8 [n_kv_heads][64];  k_sigma, v_sigma : device float [n_kv_heads][64]
 *   cache       : device, zero-initialised, regions of kvq_cache_bytes(g) bytes
 * Appends OR codes into partially filled tiles; sequences must not share regions.
 * Device-side entries with first_slot < 0, n_new < 0, n_new > max_new or
 * first_slot + n_new > capacity_tokens are skipped (nothing written for them).
 * Requirements: head_dim 128; 0 <= max_new <= capacity; k, v 4-byte aligned with
 * even strides; cache 16-byte aligned; metadata naturally aligned. */
int32_t kvq_quantize_pack(const kvq_geom *g, const void *k, const void *v, int64_t stride_tok,
                          int64_t stride_head, int32_t n_seq, const int64_t *first_slot,
                          const int32_t *n_new, const int64_t *src_row0, int32_t max_new,
                          const uint8_t *k_bits, const float *k_sigma, const float *v_sigma,
                          uint8_t *cache, const int64_t *seq_byte_off, void *stream);

/* a4 + a5 -- Packed-cache GQA decode attention (page abstract: packed-cache
 * serving path).  For sequence s and query head h (KV head h / (n_q_heads/n_kv_heads)):
 *   out[s][h] = sum_t p_t vhat_t,  p = softmax_t(softmax_scale * q[s][h] . khat_t),
 * over slots t < seq_len[s], with khat = s_t * sigma_i * level_w[code] (raw value at
 * width 16, 0 at width 0) and vhat likewise.  The token axis is split into chunks
 * whose partial (max, sum, output) are merged by a log-sum-exp combine.  Empty
 * sequences give 0.
 *   q        : device binary16 [n_seq][n_q_heads][128] (post-RoPE), contiguous
 *   seq_len  : device int32 [n_seq] (clamped to [0, max_len])
 *   out      : device float [n_seq][n_q_heads][128]
 *   workspace: device scratch of at least kvq_decode_workspace_bytes(...) bytes: the
 *              split partials, and for the vector-ALU kernel (KVQ_DECODE_GENERIC) after
 *              them a query table of n_seq * n_kv_heads * 128 * G floats (G = the group
 *              size padded to 4, 8 or 16); no initial contents are required; calls that
 *              share a workspace must not overlap in time
 * Requirements: head_dim 128; n_q_heads multiple of n_kv_heads with ratio <= 16
 * (<= 8 for KVQ_DECODE_MFMA); 0 <= max_len <= capacity; q, cache, out and
 * workspace 16-byte aligned. */
int32_t kvq_packed_decode_attn(const kvq_geom *g, int32_t n_q_heads, const void *q, const uint8_t *cache,
                               const int64_t *seq_byte_off, const int32_t *seq_len, int32_t n_seq,
                               int64_t max_len, const uint8_t *k_bits, const float *k_sigma,
                               const float *v_sigma, float softmax_scale, float *out, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Same, choosing the kernel (KVQ_DECODE_*) and the number of 64-token tiles per
 * split chunk (0 = automatic).  Returns KVQ_ERR_SHAPE if the chosen kernel cannot
 * serve the geometry. */
int32_t kvq_packed_decode_attn_ex(const kvq_geom *g, int32_t n_q_heads, const void *q, const uint8_t *cache,
                                  const int64_t *seq_byte_off, const int32_t *seq_len, int32_t n_seq,
                                  int64_t max_len, const uint8_t *k_bits, const float *k_sigma,
                                  const float *v_sigma, float softmax_scale, float *out, void *workspace,
                                  size_t workspace_bytes, int32_t kernel, int32_t tiles_per_split,
                                  void *stream);

/* Allocation-free variant of kvq_packed_decode_attn, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, meaning and result as kvq_packed_decode_attn (automatic
 * kernel and split plan) without the workspace: the split partials live in a device array
 * owned by the library, KVQ_NOALLOC_SCRATCH_BYTES bytes per GPU, reserved when the library
 * is loaded on that GPU and held until the process ends.  The call allocates nothing
 * (no hipMalloc or allocating library routine).  Returns KVQ_ERR_WORKSPACE when the plan's
 * partials (kvq_decode_workspace_bytes for the same arguments) exceed that size.  All
 * calls on one GPU share its array: calls that overlap in time on one GPU (different
 * streams, or threads without ordering) race and give undefined results; calls ordered on
 * one stream are safe.  The first call on each device looks the array up (a HIP symbol
 * query) under a lock. */
#define KVQ_NOALLOC_SCRATCH_BYTES (8u << 20)
int32_t kvq_packed_decode_attn_noalloc(const kvq_geom *g, int32_t n_q_heads, const void *q, const uint8_t *cache,
                                       const int64_t *seq_byte_off, const int32_t *seq_len, int32_t n_seq,
                                       int64_t max_len, const uint8_t *k_bits, const float *k_sigma,
                                       const float *v_sigma, float softmax_scale, float *out, void *stream);

/* The two phases of kvq_packed_decode_attn_ex, for callers that merge partials
 * themselves (e.g. partials gathered from several devices that each hold a token
 * range) or time the phases apart.
 *
 * kvq_decode_partials writes, for every (sequence s, query head h, chunk k < n_split),
 * 130 floats at partials[((s*n_q_heads + h)*n_split + k)*130]:
 *   [0] m = a reference for the chunk's logits z_t = softmax_scale * q.khat_t * log2(e):
 *           max_t z_t - 8 <= m <= max_t z_t + e (a running maximum that moves lazily,
 *           plus an integer e >= 0 taken from the value norms); -inf if the chunk is empty
 *   [1] l = sum_t 2^(z_t - m)
 *   [2..129] o_c = sum_t 2^(z_t - m) vhat_{t,c}          (unnormalised)
 * Any reference gives the same merged result: the merge weighs chunk k by 2^(m_k - M).
 * n_split is kvq_decode_n_split(...) for the same arguments; partials_bytes must be
 * at least kvq_decode_workspace_bytes_ex(...) (with KVQ_DECODE_GENERIC the bytes after
 * the partials hold that kernel's query table). */
int32_t kvq_decode_partials(const kvq_geom *g, int32_t n_q_heads, const void *q, const uint8_t *cache,
                            const int64_t *seq_byte_off, const int32_t *seq_len, int32_t n_seq, int64_t max_len,
                            const uint8_t *k_bits, const float *k_sigma, const float *v_sigma, float softmax_scale,
                            float *partials, size_t partials_bytes, int32_t kernel, int32_t tiles_per_split,
                            void *stream);
/* The decode step (the batch workload's step: each sequence appends its new token,
 * then attends all its tokens including it).  For every sequence s with
 * seq_len[s] >= 1, the rows k_new / v_new of s (element (s, h, c) at
 * base[s*new_stride_seq + h*new_stride_head + c], binary16) are quantized and packed
 * into slot seq_len[s] - 1 exactly as kvq_quantize_pack would (that slot's bits must
 * be zero), and the attention over slots [0, seq_len[s]) is computed as by
 * kvq_decode_partials / kvq_packed_decode_attn_ex.  With the matrix-core kernel the
 * append happens inside the attention kernel (the wave that owns the last tile);
 * otherwise a one-wave append kernel runs first on the same stream.  The results
 * (cache bytes, partials, out) are those of the two separate calls.
 * Requirements: those of both calls; k_new, v_new 4-byte aligned, strides even. */
int32_t kvq_decode_step_partials(const kvq_geom *g, int32_t n_q_heads, const void *q, const void *k_new,
                                 const void *v_new, int64_t new_stride_seq, int64_t new_stride_head,
                                 uint8_t *cache, const int64_t *seq_byte_off, const int32_t *seq_len,
                                 int32_t n_seq, int64_t max_len, const uint8_t *k_bits, const float *k_sigma,
                                 const float *v_sigma, float softmax_scale, float *partials,
                                 size_t partials_bytes, int32_t kernel, int32_t tiles_per_split, void *stream);
int32_t kvq_decode_step(const kvq_geom *g, int32_t n_q_heads, const void *q, const void *k_new, const void *v_new,
                        int64_t new_stride_seq, int64_t new_stride_head, uint8_t *cache,
                        const int64_t *seq_byte_off, const int32_t *seq_len, int32_t n_seq, int64_t max_len,
                        const uint8_t *k_bits, const float *k_sigma, const float *v_sigma, float softmax_scale,
                        float *out, void *workspace, size_t workspace_bytes, int32_t kernel,
                        int32_t tiles_per_split, void *stream);
/* The fp16 recent-window variant (the page's recent-key buffer: the newest tokens are
 * kept unquantized; "RoPE-Aware Bit Allocation for KV-Cache Quantization", the
 * evaluation's remark that its reasoning run keeps no such buffer).  For a sequence of
 * seq_len[s] = n tokens and a window of W tokens (1 <= W <= 1024), tokens
 * [0, max(n - W, 0)) live in the packed cache (slots 0..) and the last min(n, W)
 * tokens in a caller-owned binary16 ring: token t at row t mod W of
 *   win_k / win_v : [n_seq][n_kv_heads][W][128] binary16, 16-byte aligned.
 * kvq_window_decode_attn: attention of q over the packed tokens (dequantized, as
 *   kvq_packed_decode_attn) and the window tokens (their exact binary16 values), one
 *   softmax over all n tokens; out as kvq_packed_decode_attn.  max_len >= every
 *   seq_len[s]; the packed part needs capacity_tokens >= max_len - W, and the
 *   workspace kvq_window_workspace_bytes(...) bytes (the packed part's chunks plus one
 *   chunk for the window, computed in the same launch).  Nothing is written but out
 *   and the workspace.
 * kvq_window_decode_step: one decode step with seq_len[s] already counting the new
 *   token (rows k_new / v_new of s, as in kvq_decode_step, but 16-byte aligned with
 *   strides a multiple of 8 elements): when n > W the token leaving the window
 *   (position n - W - 1, ring row (n - 1) mod W) is quantized and packed into slot
 *   n - W - 1 exactly as kvq_quantize_pack would, inside the attention launch; the
 *   attention is that of kvq_window_decode_attn with the new token in the window;
 *   then the new token is written to ring row (n - 1) mod W.  The caller fills the
 *   ring for the prefill (tokens [n - W, n)) and quantizes the rest. */
int64_t kvq_window_workspace_bytes(const kvq_geom *g, int32_t window, int32_t n_q_heads, int32_t n_seq,
                                   int64_t max_len, int32_t kernel, int32_t tiles_per_split);
int32_t kvq_window_decode_attn(const kvq_geom *g, int32_t window, int32_t n_q_heads, const void *q,
                               const void *win_k, const void *win_v, const uint8_t *cache,
                               const int64_t *seq_byte_off, const int32_t *seq_len, int32_t n_seq, int64_t max_len,
                               const uint8_t *k_bits, const float *k_sigma, const float *v_sigma,
                               float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                               int32_t kernel, int32_t tiles_per_split, void *stream);
int32_t kvq_window_decode_step(const kvq_geom *g, int32_t window, int32_t n_q_heads, const void *q,
                               const void *k_new, const void *v_new, int64_t new_stride_seq,
                               int64_t new_stride_head, void *win_k, void *win_v, uint8_t *cache,
                               const int64_t *seq_byte_off, const int32_t *seq_len, int32_t n_seq, int64_t max_len,
                               const uint8_t *k_bits, const float *k_sigma, const float *v_sigma,
                               float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                               int32_t kernel, int32_t tiles_per_split, void *stream);
/* Chunked prefill attention over the packed cache, causal ("RoPE-Aware Bit Allocation
 * for KV-Cache Quantization", abstract: at 256K and 512K only the packed cache fits in
 * memory.  Read here as a prompt filled into it chunk by chunk, each chunk's queries
 * attending everything packed before them and their own chunk, which the caller packs
 * first with kvq_quantize_pack).
 *   q        : device binary16 [n_seq][max_q][n_q_heads][128] (post-RoPE), 16-byte aligned
 *   q_start  : device int32 [n_seq], position of sequence s's first chunk query
 *   n_q      : device int32 [n_seq], its number of queries, 0 <= n_q[s] <= max_q
 *   out      : device float [n_seq][max_q][n_q_heads][128], 16-byte aligned
 * Query j < n_q[s] of sequence s (position q_start[s] + j) attends slots
 * [0, q_start[s] + j] of the packed cache: its row of out is what
 * kvq_packed_decode_attn gives for that query at seq_len q_start[s] + j + 1 (same
 * scale, same dequantization, within the same fp32-accumulate tolerance).  Rows
 * j >= n_q[s] are written as 0.  max_len must bound every q_start[s] + n_q[s] and be
 * <= capacity_tokens (device values outside the contract are clamped so that reads
 * stay inside the sequence's region; their results are unspecified).
 * n_split: key-range splits per block of 256 query rows (0 = the planner's choice:
 * enough workgroups to fill the device, at least 8 tiles per split); with 1 the
 * attention kernel writes out itself, otherwise its partials (the decode partials'
 * format, in the workspace) are merged by kvq_merge_partials' kernel on the same
 * stream.  workspace: kvq_prefill_workspace_bytes(...) bytes (may be NULL when that is 0).
 * Served: head_dim 128 (every budget and value width, the K16 / V16 passthroughs
 * included) and n_q_heads / n_kv_heads <= 128; otherwise KVQ_ERR_SHAPE.  Any finite
 * binary16 keys and values are served: the weights entering the binary16 matrix
 * operands are scaled by a power of two chosen from the value norms seen, so no value
 * norm overflows them (the same holds for every decode call).
 * Nothing but out and the workspace is written. */
int32_t kvq_prefill_plan(const kvq_geom *g, int32_t n_q_heads, int32_t n_seq, int32_t max_q, int64_t max_len,
                         int32_t n_split, int32_t *n_split_out, int64_t *workspace_out);
int64_t kvq_prefill_workspace_bytes(const kvq_geom *g, int32_t n_q_heads, int32_t n_seq, int32_t max_q,
                                    int64_t max_len, int32_t n_split);
int32_t kvq_packed_prefill_attn(const kvq_geom *g, int32_t n_q_heads, const void *q, const uint8_t *cache,
                                const int64_t *seq_byte_off, const int32_t *q_start, const int32_t *n_q,
                                int32_t n_seq, int32_t max_q, int64_t max_len, const uint8_t *k_bits,
                                const float *k_sigma, const float *v_sigma, float softmax_scale, float *out,
                                void *workspace, size_t workspace_bytes, int32_t n_split, void *stream);
/* The TurboQuant-MSE rotation variant (TQ-MSE proper: the uniform baseline Block-GTQ
 * is measured against in "RoPE-Aware Bit Allocation for KV-Cache Quantization",
 * abstract; the related-papers page for "Quantization Dominates Rank Reduction for
 * KV-Cache" names its key path "WHT + MSE").  Each KV head has a seeded sign vector sg
 * (128 bytes: 1 = -1, 0 = +1, the caller's random draw) and the rotation
 * R = H diag(sg) / sqrt(128), H the 128 x 128 Sylvester Hadamard matrix.
 *
 * kvq_rot_quantize_pack: as kvq_quantize_pack, but every key is rotated and each of its
 *   128 rotated coordinates coded at the uniform width w = k_budget / 64 (1..8):
 *   S = H (sg * k) is formed exactly (binary16 values are integer counts of 2^-24) and
 *   rounded once to binary32, s = the token norm of the unrotated row (R keeps it), and
 *   code_i = #{ j in 1..2^w-1 : S_i >= RN32(s * thr_w[j]) }, packed in layout v1 with all
 *   block widths w.  Values: rotated and coded the same way at width v_bits when
 *   v_signs != NULL, else coded as kvq_quantize_pack does with the block scales v_sigma.
 *     k_signs, v_signs : device uint8 [n_kv_heads][128];  v_sigma : device float [n_kv_heads][64]
 *   Requirements: those of kvq_quantize_pack; k_budget a multiple of 64 in 64..512,
 *   v_bits 1..8; otherwise KVQ_ERR_BUDGET.
 * Attention over such a cache is kvq_packed_decode_attn on rotated queries with block
 * widths w everywhere, key scales sigma_rot = RN32(1/sqrt(128)) (bits KVQ_ROT_SIGMA_BITS)
 * and, for rotated values, value scales sigma_rot, followed by kvq_rot_back:
 * kvq_rot_queries: q_rot[r] = RN16(RN32(RN32(S_i) * sigma_rot)) with S = H (sg * q[r]) exact,
 *   sg the key signs of row r's KV head (query head r % n_q_heads over the group size);
 *   q, q_rot : device binary16 [n_seq][n_q_heads][128] (a rotated query must fit binary16).
 * kvq_rot_back: out[r] <- diag(sg) H out[r] / sqrt(128) in place (binary32), sg the value
 *   signs of row r's KV head: the attention output rotated back once per head. */
#define KVQ_ROT_SIGMA_BITS 0x3DB504F3u
int32_t kvq_rot_quantize_pack(const kvq_geom *g, const void *k, const void *v, int64_t stride_tok,
                              int64_t stride_head, int32_t n_seq, const int64_t *first_slot, const int32_t *n_new,
                              const int64_t *src_row0, int32_t max_new, const uint8_t *k_signs,
                              const uint8_t *v_signs, const float *v_sigma, uint8_t *cache,
                              const int64_t *seq_byte_off, void *stream);
int32_t kvq_rot_queries(const kvq_geom *g, int32_t n_q_heads, int32_t n_seq, const void *q, void *q_rot,
                        const uint8_t *k_signs, void *stream);
int32_t kvq_rot_back(const kvq_geom *g, int32_t n_q_heads, int32_t n_seq, float *out, const uint8_t *v_signs,
                     void *stream);
/* The rotated variant's decode step, first half, in one launch: each sequence's new token
 * (k_new, v_new: binary16 rows [n_seq][n_kv_heads][128] at element strides
 * new_stride_seq / new_stride_head) rotated, coded and packed into slot seq_len[s] - 1,
 * byte for byte as kvq_rot_quantize_pack packs it, and the queries rotated as
 * kvq_rot_queries rotates them (q, q_rot: [n_seq][n_q_heads][128] binary16).  Slots outside
 * [0, capacity) are skipped.  Requirements: those of kvq_rot_quantize_pack and
 * kvq_rot_queries; the slot's bytes zero before the call (appends OR into the runs);
 * n_seq and n_kv_heads + n_q_heads at most 65535 (else KVQ_ERR_SHAPE).  Errors as those
 * two calls report them; the caller owns every buffer. */
int32_t kvq_rot_decode_prepare(const kvq_geom *g, int32_t n_q_heads, int32_t n_seq, const void *q, void *q_rot,
                               const void *k_new, const void *v_new, int64_t new_stride_seq, int64_t new_stride_head,
                               uint8_t *cache, const int64_t *seq_byte_off, const int32_t *seq_len,
                               const uint8_t *k_signs, const uint8_t *v_signs, const float *v_sigma, void *stream);
/* The rotated variant's decode step, split phase, in ONE launch: what
 * kvq_rot_decode_prepare followed by kvq_decode_step_partials' attention does, with the
 * queries rotated and the new token rotated, coded and packed inside the matrix-core
 * attention kernel (no q_rot buffer, no separate launch).  q: the UNROTATED queries
 * [n_seq][n_q_heads][128]; k_new, v_new, strides: as kvq_decode_step_partials (token
 * seq_len[s] - 1 is appended, then attended); k_bits: every block at the uniform width
 * w = k_budget / 64; k_sigma: sigma_rot everywhere; v_sigma: sigma_rot (rotated values) or
 * the value block scales (values coded unrotated, v_signs == NULL, which then also code
 * the new token's values); k_signs / v_signs: as kvq_rot_quantize_pack.  The packed
 * bytes equal kvq_rot_decode_prepare's and the partials kvq_decode_partials' on the
 * rotated queries, bit for bit; merge them with kvq_merge_partials and, for rotated
 * values, rotate the output back with kvq_rot_back.  Requirements: those of
 * kvq_rot_quantize_pack's geometry and of kvq_decode_step_partials with the matrix-core
 * kernel (k_budget <= 256, GQA ratio <= 8), else KVQ_ERR_BUDGET / KVQ_ERR_SHAPE; k_signs
 * non-NULL (KVQ_ERR_ARG).  Errors as kvq_decode_step_partials reports them.  Written: the
 * new token's slot in the cache and the partials. */
int32_t kvq_rot_decode_step_partials(const kvq_geom *g, int32_t n_q_heads, const void *q, const void *k_new,
                                     const void *v_new, int64_t new_stride_seq, int64_t new_stride_head,
                                     uint8_t *cache, const int64_t *seq_byte_off, const int32_t *seq_len,
                                     int32_t n_seq, int64_t max_len, const uint8_t *k_bits, const float *k_sigma,
                                     const float *v_sigma, const uint8_t *k_signs, const uint8_t *v_signs,
                                     float softmax_scale, float *partials, size_t partials_bytes,
                                     int32_t tiles_per_split, void *stream);

/* Measurement helper (not a step of the method): a plain streaming read of `bytes`
 * (a multiple of 16; src 16-byte aligned) by n_blocks workgroups of 256 threads, each
 * writing one 32-bit word to sink[block] so the loads stay live (sink: n_blocks words).
 * Timed by the caller, it gives the read rate a simple kernel reaches on the device --
 * the ceiling the attention kernels are compared against. */
int32_t kvq_read_probe(const void *src, int64_t bytes, uint32_t *sink, int32_t n_blocks, void *stream);
/* Log-sum-exp merge of n_split partials per (sequence, head) in the format above:
 * out[s][h][c] = sum_k 2^(m_k - M) o_k,c / sum_k 2^(m_k - M) l_k, M = max_k m_k; rows
 * with no tokens give 0.  out: device float [n_seq][n_q_heads][128]. */
int32_t kvq_merge_partials(int32_t n_seq, int32_t n_q_heads, int32_t n_split, const float *partials, float *out,
                           void *stream);
/* The decode plan for these arguments: chosen kernel (KVQ_DECODE_GENERIC or
 * KVQ_DECODE_MFMA), tiles per chunk, chunks per sequence, workspace bytes.  Any
 * output pointer may be NULL.  Host only. */
int32_t kvq_decode_plan(const kvq_geom *g, int32_t n_q_heads, int32_t n_seq, int64_t max_len, int32_t kernel,
                        int32_t tiles_per_split, int32_t *kernel_out, int32_t *tiles_out, int32_t *n_split_out,
                        int64_t *workspace_out);
/* Number of chunks the decode kernels split each sequence into (negative status if invalid). */
int32_t kvq_decode_n_split(const kvq_geom *g, int32_t n_q_heads, int32_t n_seq, int64_t max_len, int32_t kernel,
                           int32_t tiles_per_split);

/* Workspace bytes needed by kvq_packed_decode_attn(_ex) (negative status if invalid). */
int64_t kvq_decode_workspace_bytes(const kvq_geom *g, int32_t n_q_heads, int32_t n_seq, int64_t max_len);
int64_t kvq_decode_workspace_bytes_ex(const kvq_geom *g, int32_t n_q_heads, int32_t n_seq, int64_t max_len,
                                      int32_t kernel, int32_t tiles_per_split);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
