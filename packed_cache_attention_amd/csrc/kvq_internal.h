// kvq_internal.h -- device helpers, constant tables and launch wrappers shared by
// the HIP translation units of libkvq.so (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"
#include "kvq_codebooks.inc"

namespace kvq {

constexpr int kTile = 64;       // token slots per tile
constexpr int kHeadDim = 128;   // head_dim served by quantize/attention
constexpr int kMaxBlocks = 64;  // d/2 for d = 128
constexpr float kLog2e = 1.4426950408889634f;

// Codebook tables in constant memory (one copy per translation unit); width w
// occupies entries [KVQ_CB_OFF(w), KVQ_CB_OFF(w) + 2^w).
static __constant__ unsigned short c_levels[510] = {KVQ_LEVELS_FP16_LIST};
static __constant__ float c_thresholds[510] = {KVQ_THRESHOLDS_LIST};
static __constant__ float c_gain_dd[8] = {KVQ_GAIN_DD_LIST};

// binary16 bit pattern -> float (exact)
__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// ---- quantization arithmetic shared by the quantize, append and fused decode kernels
// (callers compile with FP contraction off: every product here is rounded on its own)
// code = #{ j in 1..2^w-1 : x >= RN32(s * RN32(sig * thr_w[j])) }; the products are
// non-decreasing in j, so the count is found by binary lifting.
__device__ __forceinline__ uint32_t code_of(const float* thr_all, float x, int w, float sig, float s) {
#pragma clang fp contract(off)
    const float* thr = thr_all + KVQ_CB_OFF(w);
    uint32_t code = 0;
    for (int bit = 1 << (w - 1); bit >= 1; bit >>= 1) {
        const uint32_t cand = code + bit;
        const float a = sig * thr[cand];
        const float b = s * a;
        if (x >= b) code = cand;
    }
    return code;
}

__device__ __forceinline__ uint32_t encode(const float* thr_all, uint32_t bits16, int w, float sig, float s) {
    if (w == 0) return 0;
    if (w == 16) return bits16;
    return code_of(thr_all, h2f(bits16), w, sig, s);
}

// balanced pairwise binary32 tree over the 128 squares (lane l: coordinates 2l, 2l+1)
__device__ __forceinline__ float token_norm(uint32_t pair) {
#pragma clang fp contract(off)
    const float a = h2f(pair & 0xffffu), b = h2f(pair >> 16);
    float t = a * a + b * b;  // both squares exact in binary32
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) t = t + __shfl_xor(t, m);
    return sqrtf(t);  // correctly rounded on gfx950
}

// ---- layout ----
__host__ __device__ inline int64_t k_record_bytes(int k_budget) { return 16 * ((2 * (int64_t)k_budget + 127) / 128); }
__host__ __device__ inline int64_t tile_bytes(int d, int k_budget, int v_bits) {
    return kTile * k_record_bytes(k_budget) + (int64_t)d * 8 * v_bits + 2 * kTile * 4;
}

// ---- launch wrappers (host side, one per kernel family) ----
hipError_t launch_block_energy(const uint16_t* x, int64_t n_tok, int64_t stride_tok, int64_t stride_head,
                               int n_heads, int d, int pairing, uint64_t* energy, hipStream_t st);
hipError_t launch_allocate(const uint64_t* energy, int n_units, int nb, int budget, int mode, uint8_t* bits,
                           float* sigma, hipStream_t st);
hipError_t launch_quantize_pack(const kvq_geom& g, const uint16_t* k, const uint16_t* v, int64_t stride_tok,
                                int64_t stride_head, int n_seq, const int64_t* first_slot, const int32_t* n_new,
                                const int64_t* src_row0, int max_new, const uint8_t* k_bits, const float* k_sigma,
                                const float* v_sigma, uint8_t* cache, const int64_t* seq_byte_off, hipStream_t st);

// The decode step's new token per sequence (row s at k + s*stride_seq + h*stride_head),
// written to slot seq_len[s] - 1 before attention; k == nullptr: no append.
// window > 0 (the fp16 recent window): the packed cache holds the first
// seq_len[s] - window tokens, attention reads only those, and the appended token is
// the one leaving the window -- row ((seq_len[s] - 1) mod window) of the ring at
// k + s*stride_seq + h*stride_head, written to packed slot seq_len[s] - window - 1.
struct AppendArgs {
    const uint16_t* k;
    const uint16_t* v;
    int64_t stride_seq;
    int64_t stride_head;
    int32_t window;
};

struct DecodePlan {
    int kernel;           // KVQ_DECODE_GENERIC or KVQ_DECODE_MFMA
    int tiles_per_split;  // 64-token tiles per chunk
    int n_split;          // chunks per (sequence, KV head)
    int64_t workspace;    // bytes
};
// Returns 0 and fills the plan, or a negative kvq_status.
int plan_decode(const kvq_geom& g, int n_q_heads, int n_seq, int64_t max_len, int kernel, int tiles_per_split,
                DecodePlan* plan);
hipError_t launch_decode_partials(const kvq_geom& g, const DecodePlan& plan, int n_q_heads, const uint16_t* q,
                                  uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len,
                                  int n_seq, int64_t max_len, const uint8_t* k_bits, const float* k_sigma,
                                  const float* v_sigma, float softmax_scale, float* partials, hipStream_t st,
                                  const AppendArgs& app = AppendArgs{nullptr, nullptr, 0, 0, 0});
// one token per sequence into slot seq_len[s] - 1 (the decode step's append, alone)
hipError_t launch_append_step(const kvq_geom& g, int n_seq, const AppendArgs& app, const int32_t* seq_len,
                              const uint8_t* k_bits, const float* k_sigma, const float* v_sigma, uint8_t* cache,
                              const int64_t* seq_byte_off, hipStream_t st);
hipError_t launch_merge(int n_rows, int n_split, const float* partials, float* out, hipStream_t st);
// the split merge of the packed part folded with exact attention over the fp16 window
// (ring [n_seq][n_kv][window][128]); with k_new, the step's new token is read from
// k_new/v_new and written to its ring row after use
struct WindowArgs {
    const uint16_t* q;
    int n_q, g, n_kv, window;
    float scale_log2;
    uint16_t* win_k;
    uint16_t* win_v;
    const int32_t* seq_len;
    const uint16_t* k_new;
    const uint16_t* v_new;
    int64_t new_stride_seq, new_stride_head;
};
hipError_t launch_merge_window(int n_seq, int n_split, const float* partials, float* out, const WindowArgs& w,
                               hipStream_t st);

}  // namespace kvq
