// kvq_quantize.hip -- per-token norm, Lloyd-Max codes at the allocated widths and
// bit packing into 64-slot tiles (packed layout v1), for "RoPE-Aware Bit
// Allocation for KV-Cache Quantization" (abstract: TQ-MSE codes at the widths the
// Block-GTQ allocator assigns, kept in a packed cache).
//
// One workgroup owns one (sequence, KV head, tile): it is the only writer of that
// tile during the call, so partially filled tiles are updated with plain
// read-modify-write.  Phase 1: each wave takes tokens; lane l holds coordinates
// 2l, 2l+1, forms the squared-norm tree with xor-butterflies (level 1 is the
// lane's own pair, level k the butterfly with mask 2^(k-2)), and finds each code
// by binary search over the monotone threshold products.  Phase 2: the tile's K
// records, V runs and scales are assembled dword by dword from the codes in LDS.
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {

// Bulk quantize + pack, one workgroup per (sequence, KV head, tile), lane = token.
// The tile's fp16 rows are staged in LDS (rows 65 dwords apart: a coordinate read
// by 64 lanes touches distinct banks).  Norms: waves 0-3 sum the four 16-pair
// quarters of each K row, waves 4-7 those of V.  Codes: each wave takes a run of
// K-order fields (about an eighth of the work) and 16 of the V coordinates.  A
// field's width is the same for every lane, so the binary lifting runs without
// divergence, several fields side by side.  Each coordinate is read by one wave
// only, which overwrites its fp16 value with the code; the store phase then builds
// every K record word and V run word in one thread from those code rows.
constexpr int kRowDw = kHeadDim / 2 + 1;
constexpr int kQWaves = 8;  // waves per workgroup
constexpr int kQThreads = 64 * kQWaves;
constexpr int kGroup = 4;   // K fields searched side by side
constexpr int kVGroup = 8;  // V coordinates searched side by side

// LDS byte address of a shared-memory object
typedef __attribute__((address_space(3))) const float lds_cf32;
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_cf32*)p; }

// One step of binary lifting on threshold addresses: `at` is the LDS byte address of
// the threshold of the code found so far (the table start for code 0); the candidate
// lies `inc` bytes further (4 << open bit position).  The step moves to the candidate
// when the value reaches its product RN(s * RN(sig * t)); a NaN threshold never does.
__device__ __forceinline__ uint32_t lift(uint32_t at, uint32_t inc, float x, float sig, float s) {
    const uint32_t c = at + inc;
    const float a = *(lds_cf32*)(uintptr_t)c;
    const float b = s * (sig * a);
    return x >= b ? c : at;
}

__global__ __launch_bounds__(kQThreads) void quantize_pack_kernel(
    const uint16_t* __restrict__ kx, const uint16_t* __restrict__ vx, int64_t stride_tok, int64_t stride_head,
    const int64_t* __restrict__ first_slot, const int32_t* __restrict__ n_new, const int64_t* __restrict__ src_row0,
    int max_new, int64_t capacity, const uint8_t* __restrict__ k_bits, const float* __restrict__ k_sigma,
    const float* __restrict__ v_sigma, uint8_t* __restrict__ cache, const int64_t* __restrict__ seq_byte_off,
    int pairing, int k_budget, int v_bits) {
    const int s = blockIdx.z, h = blockIdx.y;
    const int64_t first = first_slot[s];
    const int n = n_new[s];
    if (first < 0 || n <= 0 || n > max_new || first + n > capacity) return;
    const int64_t tau = first / kTile + blockIdx.x;
    const int64_t tile0 = tau * kTile;
    const int64_t lo_slot = max(first, tile0), hi_slot = min(first + (int64_t)n, tile0 + kTile);
    if (lo_slot >= hi_slot) return;
    const int lo_p = (int)(lo_slot - tile0), hi_p = (int)(hi_slot - tile0);

    const int64_t SK = k_record_bytes(k_budget);
    const int64_t TB = tile_bytes(kHeadDim, k_budget, v_bits);
    const int RW = (int)(SK / 4);  // words per K record
    const int VW = 2 * v_bits;     // words per V run
    uint8_t* tile = cache + seq_byte_off[s] + ((int64_t)h * (capacity / kTile) + tau) * TB;

    __shared__ uint32_t s_k[kTile * kRowDw], s_v[kTile * kRowDw];
    __shared__ float s_thr[512];  // the codebook thresholds, then a NaN
    __shared__ float s_quarter[kQWaves][kTile];
    __shared__ float s_ks[kTile], s_vs[kTile];
    // K order, field f: coordinate | width << 7 | bit offset << 12, and the block's
    // sigma; padded so that a group read from any f stays in the arrays
    __shared__ uint32_t s_fx[kHeadDim + kGroup];
    __shared__ float s_fsig[kHeadDim + kGroup];
    __shared__ float s_vsig[kHeadDim];
    __shared__ int s_range[kQWaves + 1];  // wave w encodes fields [s_range[w], s_range[w+1])
    __shared__ uint8_t s_wfirst[64];      // the field holding bit 32k of the record (nf: none)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform in the wave

    // ---- phase 0: rows, thresholds, K order
    const int64_t row0 = src_row0[s] + (tile0 - first);  // source row of slot 0 (only rows of valid slots are read)
    const uint16_t* ksrc = kx + (int64_t)h * stride_head;
    const uint16_t* vsrc = vx + (int64_t)h * stride_head;
    if ((((uintptr_t)kx | (uintptr_t)vx) & 15) == 0 && ((stride_tok | stride_head) & 7) == 0) {
        const int j = tid & 15;  // 16-byte piece of a 256-byte row
#pragma unroll
        for (int i = 0; i < kTile * 16 / kQThreads; ++i) {
            const int p = (tid >> 4) + (kQThreads / 16) * i;
            if (p >= lo_p && p < hi_p) {
                const uint4 a = *(const uint4*)(ksrc + (row0 + p) * stride_tok + 8 * j);
                const uint4 b = *(const uint4*)(vsrc + (row0 + p) * stride_tok + 8 * j);
                uint32_t* dk = s_k + p * kRowDw + 4 * j;
                uint32_t* dv = s_v + p * kRowDw + 4 * j;
                dk[0] = a.x; dk[1] = a.y; dk[2] = a.z; dk[3] = a.w;
                dv[0] = b.x; dv[1] = b.y; dv[2] = b.z; dv[3] = b.w;
            }
        }
    } else {  // rows only 4-byte aligned: one coordinate pair per lane
        for (int p = wave; p < hi_p; p += kQWaves) {
            if (p < lo_p) continue;
            s_k[p * kRowDw + lane] = *(const uint32_t*)(ksrc + (row0 + p) * stride_tok + 2 * lane);
            s_v[p * kRowDw + lane] = *(const uint32_t*)(vsrc + (row0 + p) * stride_tok + 2 * lane);
        }
    }
    for (int i = tid; i < 510; i += kQThreads) s_thr[i] = c_thresholds[i];
    if (tid == 0) s_thr[510] = __builtin_nanf("");
    if (tid < kHeadDim) {
        const int blk = pairing == KVQ_PAIR_HALF ? (tid & (kMaxBlocks - 1)) : (tid >> 1);
        s_vsig[tid] = v_sigma[h * kMaxBlocks + blk];
    }
    if (tid < kMaxBlocks) {
        // rank blocks by (width desc, index asc); a block's fields p, q follow every
        // wider block and the lower-indexed blocks of its own width
        const int i = tid;
        const int w = k_bits[h * kMaxBlocks + i];
        const float sig = k_sigma[h * kMaxBlocks + i];
        const unsigned long long below = (1ull << i) - 1ull;
        int rank = 0, off = 0;
        for (int wc = 16; wc >= 1; --wc) {
            const unsigned long long mk = __ballot(w == wc);
            if (wc > w) { rank += __popcll(mk); off += 2 * wc * __popcll(mk); }
            if (wc == w) { rank += __popcll(mk & below); off += 2 * wc * __popcll(mk & below); }
        }
        const int nf = 2 * __popcll(__ballot(w > 0));
        s_wfirst[i] = (uint8_t)nf;
        if (w > 0) {
            const int pc = pairing == KVQ_PAIR_HALF ? i : 2 * i;
            const int qc = pairing == KVQ_PAIR_HALF ? i + kMaxBlocks : 2 * i + 1;
            s_fx[2 * rank] = pc | w << 7 | off << 12;
            s_fx[2 * rank + 1] = qc | w << 7 | (off + w) << 12;
            s_fsig[2 * rank] = s_fsig[2 * rank + 1] = sig;
            // a word boundary inside a field (at most one: w <= 16) names its first field
            const int kp = (off + 31) >> 5, kq = (off + w + 31) >> 5;
            if (32 * kp < off + w) s_wfirst[kp] = (uint8_t)(2 * rank);
            if (32 * kq < off + 2 * w) s_wfirst[kq] = (uint8_t)(2 * rank + 1);
        }
        if (i < kGroup) { s_fx[kHeadDim + i] = 0u; s_fsig[kHeadDim + i] = 0.f; }
        // split the fields into runs of about an eighth of the work each, a field of
        // width w costing about w + 2 lifting steps (its steps plus its share of the
        // per-group work); run v starts at the first field whose cost prefix reaches
        // v/8 of the total.  Field 2r (p) has prefix off + 4r, field 2r + 1 (q) has
        // off + w + 4r + 2.
        int wsum = w;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) wsum += __shfl_xor(wsum, m);
        const int total = 2 * wsum + 2 * nf;
        for (int wv = 0; wv <= kQWaves; ++wv) {
            const int bound = (int)(((int64_t)total * wv + kQWaves - 1) / kQWaves);
            const unsigned long long pb = __ballot(w > 0 && off + 4 * rank < bound);
            const unsigned long long qb = __ballot(w > 0 && off + w + 4 * rank + 2 < bound);
            if (i == 0) s_range[wv] = wv == kQWaves ? nf : __popcll(pb) + __popcll(qb);
        }
    }
    __syncthreads();

    // ---- phase 1: token norms (lane = token).  Waves 0-3 sum the squares of the K
    // row's four 32-coordinate quarters, waves 4-7 those of V, each as the pairwise
    // tree over its 16 coordinate pairs; the root adds them as (Q0 + Q1) + (Q2 + Q3),
    // which is the balanced tree over all 64 pairs.
    {
        const uint32_t* rows = wave < 4 ? s_k : s_v;
        const uint32_t* r = rows + lane * kRowDw + 16 * (wave & 3);
        float t[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint32_t pr = r[k];
            const float a = h2f(pr & 0xffffu), b = h2f(pr >> 16);
            t[k] = a * a + b * b;
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1)
#pragma unroll
            for (int k = 0; k < 16; k += 2 * m) t[k] = t[k] + t[k + m];
        s_quarter[wave][lane] = t[0];
    }
    __syncthreads();
    if (tid < 2 * kTile) {
        const int p = tid & (kTile - 1), q0 = tid < kTile ? 0 : 4;
        const float r = sqrtf((s_quarter[q0][p] + s_quarter[q0 + 1][p]) + (s_quarter[q0 + 2][p] + s_quarter[q0 + 3][p]));
        if (tid < kTile) s_ks[p] = r;
        else s_vs[p] = r;
    }
    __syncthreads();

    // ---- phase 2: codes (lane = token), written over the lane's own fp16 values
    const bool valid = lane >= lo_p && lane < hi_p;
    {
        // K: groups of kGroup consecutive fields.  Widths fall along the K order, so
        // the group's first searched field is its widest (w0); a field of width w joins
        // the lifting for its last w steps, where the open bit position is the same for
        // every field of the group.  Width-16 fields keep the raw fp16 bits.
        const float sk = s_ks[lane];
        uint16_t* krow = (uint16_t*)(s_k + lane * kRowDw);
        const int f0 = __builtin_amdgcn_readfirstlane(s_range[wave]);
        const int f1 = __builtin_amdgcn_readfirstlane(s_range[wave + 1]);
        const uint32_t thr0 = lds_addr(s_thr), nan_at = thr0 + 4u * 510u;
        for (int f = f0; f < f1; f += kGroup) {
            const int gn = min(kGroup, f1 - f);
            uint32_t fx[kGroup], at[kGroup], tb[kGroup];
            int ws[kGroup];  // search width (0: no search)
            int w0 = 0;
            float x[kGroup], sg[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                fx[i] = __builtin_amdgcn_readfirstlane(s_fx[f + i]);
                sg[i] = s_fsig[f + i];
                const int w = (fx[i] >> 7) & 31;
                ws[i] = i < gn && w != 16 ? w : 0;
                w0 = max(w0, ws[i]);
                x[i] = h2f(krow[fx[i] & 127]);
                tb[i] = thr0 + 4u * KVQ_CB_OFF(ws[i]);
                at[i] = tb[i];
            }
            // a field with fewer than w0 bits waits at its table start, its candidate
            // being the NaN, until its own top bit comes up
            for (int sh = w0 - 1; sh >= 0; --sh) {
#pragma unroll
                for (int i = 0; i < kGroup; ++i) at[i] = lift(at[i], sh < ws[i] ? 4u << sh : nan_at - tb[i], x[i], sg[i], sk);
            }
#pragma unroll
            for (int i = 0; i < kGroup; ++i)
                if (ws[i] > 0) krow[fx[i] & 127] = (uint16_t)((at[i] - tb[i]) >> 2);
        }

        // V: kVGroup coordinates at a time; slots outside the call get code 0 (16-bit
        // V keeps the raw rows, whose invalid slots the run builder skips)
        if (v_bits != 16) {
            const float sv = s_vs[lane];
            uint16_t* vrow = (uint16_t*)(s_v + lane * kRowDw);
            const uint32_t vthr = thr0 + 4u * KVQ_CB_OFF(v_bits);
            constexpr int kVPer = kHeadDim / kQWaves;
            for (int c0 = kVPer * wave; c0 < kVPer * wave + kVPer; c0 += kVGroup) {
                uint32_t at[kVGroup];
                float x[kVGroup], sg[kVGroup];
#pragma unroll
                for (int i = 0; i < kVGroup; ++i) {
                    x[i] = h2f(vrow[c0 + i]);
                    sg[i] = s_vsig[c0 + i];
                    at[i] = vthr;
                }
                for (int sh = v_bits - 1; sh >= 0; --sh) {
#pragma unroll
                    for (int i = 0; i < kVGroup; ++i) at[i] = lift(at[i], 4u << sh, x[i], sg[i], sv);
                }
#pragma unroll
                for (int i = 0; i < kVGroup; ++i) vrow[c0 + i] = valid ? (uint16_t)((at[i] - vthr) >> 2) : (uint16_t)0;
            }
        }
    }
    __syncthreads();

    // ---- phase 3: the tile's records (valid slots), runs and scales
    // K record word k of slot `lane`: the fields from s_wfirst[k] on that start
    // before bit 32k + 32, each field's code shifted to its offset
    uint32_t* krec = (uint32_t*)tile;
    {
        const uint16_t* krow = (const uint16_t*)(s_k + lane * kRowDw);
        const int nf = __builtin_amdgcn_readfirstlane(s_range[kQWaves]);
        for (int k = wave; k < RW; k += kQWaves) {
            const int lo = 32 * k;
            uint32_t val = 0u;
            int f = __builtin_amdgcn_readfirstlane(s_wfirst[k]);
            if (f < nf) {
                // the field holding bit 32k starts at or before it; the rest start inside
                const uint32_t fx0 = __builtin_amdgcn_readfirstlane(s_fx[f]);
                val = (uint32_t)krow[fx0 & 127] >> (lo - (int)((fx0 >> 12) & 2047));
                bool done = false;
                for (++f; f < nf && !done; f += kGroup) {
                    uint32_t fx[kGroup], code[kGroup];
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) fx[i] = __builtin_amdgcn_readfirstlane(s_fx[f + i]);
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) code[i] = krow[fx[i] & 127];
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) {
                        const int of = (fx[i] >> 12) & 2047;
                        if (f + i >= nf || of >= lo + 32) done = true;
                        if (!done) val |= code[i] << (of - lo);
                    }
                }
            }
            if (valid) krec[lane * RW + k] = val;
        }
    }
    const bool whole = lo_p == 0 && hi_p == kTile;
    uint32_t* vrun = (uint32_t*)(tile + kTile * SK);
    // one thread per run word; a wave's 64 lanes take one word index k of 64
    // coordinates, so the slots involved are the same in every lane and the code
    // reads of one slot are 64 neighbouring bytes
    for (int idx = tid; idx < kHeadDim * VW; idx += kQThreads) {
        const int c = idx & (kHeadDim - 1), k = __builtin_amdgcn_readfirstlane(idx >> 7);
        uint32_t val = 0u;
        if (v_bits == 16) {
            const uint16_t* col = (const uint16_t*)s_v + c;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int p = 2 * k + e;
                if (p >= lo_p && p < hi_p) val |= (uint32_t)col[p * 2 * kRowDw] << (16 * e);
            }
        } else {
            // word k holds bits [32k, 32k + 32): slots plo..phi, slot p at bit p*v_bits - 32k
            const int plo = 32 * k / v_bits, phi = min(kTile - 1, (32 * k + 31) / v_bits);
            const uint16_t* col = (const uint16_t*)s_v + c;
            const int sh0 = plo * v_bits - 32 * k;  // in (-v_bits, 0]
            val = (uint32_t)col[plo * 2 * kRowDw] >> -sh0;
            for (int p = plo + 1; p <= phi; ++p) val |= (uint32_t)col[p * 2 * kRowDw] << (p * v_bits - 32 * k);
        }
        uint32_t* dst = vrun + c * VW + k;
        if (whole) *dst = val;
        else if (val) *dst |= val;
    }
    float* scl = (float*)(tile + kTile * SK + kHeadDim * 8 * v_bits);
    if (tid >= lo_p && tid < hi_p) {
        scl[tid] = s_ks[tid];
        scl[kTile + tid] = s_vs[tid];
    }
}

// Appends of a few tokens (the decode step's new row): one wave per (token, head,
// sequence), so each call costs one round trip to memory instead of a tile pass.
// Lane l encodes coordinates 2l, 2l+1 (the norm tree pairs) and ranks block l
// for the K order; the record is OR-assembled in LDS and stored whole, and the
// V codes are OR-ed into their runs with no-return atomics (the slot's bits are
// zero in a zero-initialised cache, and concurrent tokens touch different bits).
constexpr int kAppendMax = 4;

__global__ __launch_bounds__(64) void append_kernel(
    const uint16_t* __restrict__ kx, const uint16_t* __restrict__ vx, int64_t stride_tok, int64_t stride_head,
    const int64_t* __restrict__ first_slot, const int32_t* __restrict__ n_new, const int64_t* __restrict__ src_row0,
    int max_new, int64_t capacity, const uint8_t* __restrict__ k_bits, const float* __restrict__ k_sigma,
    const float* __restrict__ v_sigma, uint8_t* __restrict__ cache, const int64_t* __restrict__ seq_byte_off,
    int pairing, int k_budget, int v_bits, const int32_t* __restrict__ step_len, AppendArgs app) {
    const int s = blockIdx.z, h = blockIdx.y, j = blockIdx.x;
    const int window = app.window;
    // either explicit runs (first_slot, n_new, src_row0) or the decode step: one token
    // per sequence, row s, into slot step_len[s] - 1; with an fp16 window of `window`
    // tokens, the token leaving it (ring row (step_len[s] - 1) mod window of row s)
    // into slot step_len[s] - window - 1
    const int64_t first = step_len ? (int64_t)step_len[s] - 1 - window : first_slot[s];
    const int n = step_len ? 1 : n_new[s];
    if (first < 0 || n <= 0 || n > max_new || first + n > capacity || j >= n) return;
    const int lane = threadIdx.x;
    const int64_t slot = first + j;
    const int64_t row = step_len ? (int64_t)s : src_row0[s] + j;
    const int64_t ring_row = window > 0 ? ((int64_t)step_len[s] - 1) % window * kHeadDim : 0;  // first >= 0 here
    const int64_t tau = slot / kTile;
    const int p = (int)(slot - tau * kTile);
    const int64_t SK = k_record_bytes(k_budget);
    const int64_t TB = tile_bytes(kHeadDim, k_budget, v_bits);
    uint8_t* tile = cache + seq_byte_off[s] + ((int64_t)h * (capacity / kTile) + tau) * TB;

    __shared__ float s_thr[510];
    __shared__ uint16_t s_fo[kHeadDim];  // bit offset of coordinate c's field in the record
    __shared__ uint32_t s_rec[64];       // the slot's K record (at most 2048 bits)

    // every load of the call is issued here, before anything waits
    const int c0 = 2 * lane, c1 = 2 * lane + 1;
    const int b0 = pairing == KVQ_PAIR_HALF ? (c0 & (kMaxBlocks - 1)) : (c0 >> 1);
    const int b1 = pairing == KVQ_PAIR_HALF ? (c1 & (kMaxBlocks - 1)) : (c1 >> 1);
    const uint32_t kp = *(const uint32_t*)(kx + row * stride_tok + (int64_t)h * stride_head + ring_row + c0);
    const uint32_t vp = *(const uint32_t*)(vx + row * stride_tok + (int64_t)h * stride_head + ring_row + c0);
    const int w0 = k_bits[h * kMaxBlocks + b0], w1 = k_bits[h * kMaxBlocks + b1];
    const float ks0 = k_sigma[h * kMaxBlocks + b0], ks1 = k_sigma[h * kMaxBlocks + b1];
    const float vs0 = v_sigma[h * kMaxBlocks + b0], vs1 = v_sigma[h * kMaxBlocks + b1];
    const int wl = k_bits[h * kMaxBlocks + lane];  // block `lane`, for the K order
    float thr[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) thr[k] = 64 * k + lane < 510 ? c_thresholds[64 * k + lane] : 0.f;

#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (64 * k + lane < 510) s_thr[64 * k + lane] = thr[k];
    s_rec[lane] = 0;
    // K order: rank of block `lane` by (width desc, index asc); its fields p, q follow
    // all wider blocks and the lower-indexed blocks of its own width
    {
        const unsigned long long below = (1ull << lane) - 1ull;
        int off = 0;
        for (int wc = 16; wc >= 1; --wc) {
            const unsigned long long mk = __ballot(wl == wc);
            if (wc > wl) off += 2 * wc * __popcll(mk);
            if (wc == wl) off += 2 * wc * __popcll(mk & below);
        }
        const int pc = pairing == KVQ_PAIR_HALF ? lane : 2 * lane;
        const int qc = pairing == KVQ_PAIR_HALF ? lane + kMaxBlocks : 2 * lane + 1;
        s_fo[pc] = (uint16_t)off;
        s_fo[qc] = (uint16_t)(off + wl);
    }
    const float sk = token_norm(kp), sv = token_norm(vp);
    __syncthreads();
    const uint32_t kc0 = encode(s_thr, kp & 0xffffu, w0, ks0, sk);
    const uint32_t kc1 = encode(s_thr, kp >> 16, w1, ks1, sk);
    const uint32_t vc0 = encode(s_thr, vp & 0xffffu, v_bits, vs0, sv);
    const uint32_t vc1 = encode(s_thr, vp >> 16, v_bits, vs1, sv);
    // K record: fields OR-ed into LDS words, then stored whole
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int w = e ? w1 : w0;
        if (w == 0) continue;
        const uint32_t code = e ? kc1 : kc0;
        const int off = s_fo[e ? c1 : c0];
        const int k = off >> 5, sh = off & 31;
        atomicOr(&s_rec[k], code << sh);
        if (sh + w > 32) atomicOr(&s_rec[k + 1], code >> (32 - sh));
    }
    __syncthreads();
    if (lane < (int)(SK / 4)) ((uint32_t*)(tile + (int64_t)p * SK))[lane] = s_rec[lane];
    // V codes into their runs (run of coordinate c: 8*v_bits bytes, slot p at bit p*v_bits)
    uint32_t* vrun = (uint32_t*)(tile + kTile * SK);
    const int vb = p * v_bits, vk = vb >> 5, vsh = vb & 31;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const uint32_t code = e ? vc1 : vc0;
        uint32_t* run = vrun + (e ? c1 : c0) * 2 * v_bits;
        if (code == 0) continue;
        atomicOr(run + vk, code << vsh);
        if (vsh + v_bits > 32 && (code >> (32 - vsh)) != 0) atomicOr(run + vk + 1, code >> (32 - vsh));
    }
    if (lane == 0) {
        float* scl = (float*)(tile + kTile * SK + kHeadDim * 8 * v_bits);
        scl[p] = sk;
        scl[kTile + p] = sv;
    }
    if (window > 0 && app.k_new != nullptr) {  // the step's new token takes the ring row just read
        const int64_t nr = (int64_t)s * app.new_stride_seq + (int64_t)h * app.new_stride_head + c0;
        const uint32_t kn = *(const uint32_t*)(app.k_new + nr);
        const uint32_t vn = *(const uint32_t*)(app.v_new + nr);
        const int64_t rr = row * stride_tok + (int64_t)h * stride_head + ring_row + c0;
        *(uint32_t*)(app.ring_k + rr) = kn;
        *(uint32_t*)(app.ring_v + rr) = vn;
    }
}

hipError_t launch_quantize_pack(const kvq_geom& g, const uint16_t* k, const uint16_t* v, int64_t stride_tok,
                                int64_t stride_head, int n_seq, const int64_t* first_slot, const int32_t* n_new,
                                const int64_t* src_row0, int max_new, const uint8_t* k_bits, const float* k_sigma,
                                const float* v_sigma, uint8_t* cache, const int64_t* seq_byte_off, hipStream_t st) {
    if (max_new <= kAppendMax) {
        dim3 grid(max_new, g.n_kv_heads, n_seq);
        hipLaunchKernelGGL(append_kernel, grid, dim3(64), 0, st, k, v, stride_tok, stride_head, first_slot, n_new,
                           src_row0, max_new, g.capacity_tokens, k_bits, k_sigma, v_sigma, cache, seq_byte_off,
                           g.rope_pairing, g.k_budget, g.v_bits, (const int32_t*)nullptr, AppendArgs{});
        return hipGetLastError();
    }
    // a run of max_new slots starting anywhere touches at most ceil(max_new/64) + 1 tiles
    const int tiles = (max_new + kTile - 1) / kTile + 1;
    dim3 grid(tiles, g.n_kv_heads, n_seq);
    hipLaunchKernelGGL(quantize_pack_kernel, grid, dim3(kQThreads), 0, st, k, v, stride_tok, stride_head, first_slot,
                       n_new, src_row0, max_new, g.capacity_tokens, k_bits, k_sigma, v_sigma, cache, seq_byte_off,
                       g.rope_pairing, g.k_budget, g.v_bits);
    return hipGetLastError();
}

hipError_t launch_append_step(const kvq_geom& g, int n_seq, const AppendArgs& app, const int32_t* seq_len,
                              const uint8_t* k_bits, const float* k_sigma, const float* v_sigma, uint8_t* cache,
                              const int64_t* seq_byte_off, hipStream_t st) {
    dim3 grid(1, g.n_kv_heads, n_seq);
    hipLaunchKernelGGL(append_kernel, grid, dim3(64), 0, st, app.k, app.v, app.stride_seq, app.stride_head,
                       (const int64_t*)nullptr, (const int32_t*)nullptr, (const int64_t*)nullptr, 1,
                       g.capacity_tokens, k_bits, k_sigma, v_sigma, cache, seq_byte_off, g.rope_pairing, g.k_budget,
                       g.v_bits, seq_len, app);
    return hipGetLastError();
}

}  // namespace kvq
