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

// ---- cross-lane helpers (DPP within a row of 16 lanes, permlane swaps across rows)
__device__ __forceinline__ float dpp_ror8(float x) {
    // row_ror:8 within each row of 16 lanes: lane l receives lane l ^ 8
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
}

// permlane{16,32}_swap(x, x) returns the even rows (halves) of x in its first result
// and the odd ones in its second: lane l sees x at l & ~16 (~32) and at l | 16 (| 32).
// The two results are copied into named integers before any bit cast (a bit cast
// applied directly to the second element reads the first).
__device__ __forceinline__ void pair16(float x, float& a, float& b) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void pair32(float x, float& a, float& b) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    a = __builtin_bit_cast(float, r0);
    b = __builtin_bit_cast(float, r1);
}
// max / sum of the value in lanes l and l ^ 16 (l ^ 32); both lanes get the same result
__device__ __forceinline__ float xor16_max(float x) { float a, b; pair16(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float xor32_max(float x) { float a, b; pair32(x, a, b); return fmaxf(a, b); }
__device__ __forceinline__ float xor16_sum(float x) { float a, b; pair16(x, a, b); return a + b; }
__device__ __forceinline__ float xor32_sum(float x) { float a, b; pair32(x, a, b); return a + b; }
// lane l ^ 1 and l ^ 2 (quad permutations) and l ^ 4 (half-row mirror: after the quad
// steps every lane of a quad holds the same value, and lane 7 - l is in the other quad)
__device__ __forceinline__ float dpp_xor1(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_mirror8(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false));
}
// maximum / sum over the 64 lanes of a wave, in every lane
__device__ __forceinline__ float wave_max64(float x) {
    x = fmaxf(x, dpp_xor1(x));
    x = fmaxf(x, dpp_xor2(x));
    x = fmaxf(x, dpp_mirror8(x));
    x = fmaxf(x, dpp_ror8(x));
    return xor32_max(xor16_max(x));
}
__device__ __forceinline__ float wave_sum64(float x) {
    x = x + dpp_xor1(x);
    x = x + dpp_xor2(x);
    x = x + dpp_mirror8(x);
    x = x + dpp_ror8(x);
    return xor32_sum(xor16_sum(x));
}

// ---- the rotated variant's exact transform (shared by its quantizer and the fused
// decode step): binary16 values are integer counts of 2^-24, so the Walsh-Hadamard sums
// of a row are exact in 64-bit integers and get one binary32 rounding
constexpr float kRotSigma = 0.0883883461356163f;  // RN32(1 / sqrt(128)): bits 0x3DB504F3
static_assert(__builtin_bit_cast(uint32_t, kRotSigma) == 0x3DB504F3u, "rotation scale");

// value of a binary16 pattern in units of 2^-24 (exact)
__device__ __forceinline__ int64_t h2units(uint32_t h) {
    const int e = (h >> 10) & 31, m = h & 1023;
    const int64_t v = e == 0 ? (int64_t)m : ((int64_t)(1024 + m) << (e - 1));
    return (h & 0x8000u) ? -v : v;
}

// lane l receives x of lane l ^ M: DPP inside each row of 16 lanes for M = 1, 2, 4, 8
// (quad permutations; for 4 two row rotates, by 12 on banks 0 and 2 and by 4 on banks 1
// and 3; a rotate by 8), permlane swaps across rows for 16 and 32 -- no LDS traffic
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int lane) {
    static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane distance");
    if constexpr (M == 1) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false);
    if constexpr (M == 2) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false);
    if constexpr (M == 4) {
        const int t = __builtin_amdgcn_update_dpp(0, (int)x, 0x12C, 0xf, 0x5, false);
        return (uint32_t)__builtin_amdgcn_update_dpp(t, (int)x, 0x124, 0xf, 0xA, false);
    }
    if constexpr (M == 8) return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xf, 0xf, false);
    if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        const uint32_t r0 = r[0], r1 = r[1];
        return (lane & 16) ? r0 : r1;
    }
    if constexpr (M == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        const uint32_t r0 = r[0], r1 = r[1];
        return (lane & 32) ? r0 : r1;
    }
    return x;
}
template <int M>
__device__ __forceinline__ int64_t lane_xor64(int64_t v, int lane) {
    const uint32_t lo = lane_xor<M>((uint32_t)v, lane), hi = lane_xor<M>((uint32_t)((uint64_t)v >> 32), lane);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
template <int M>
__device__ __forceinline__ void fwht64_stage(int64_t& a, int64_t& b, int lane) {
    const int64_t pa = lane_xor64<M>(a, lane), pb = lane_xor64<M>(b, lane);
    const bool upper = lane & M;  // this lane holds the second member of each pair
    a = upper ? pa - a : a + pa;
    b = upper ? pb - b : b + pb;
}

// The Walsh-Hadamard transform of the 128 values a wave holds, in place, exact in
// 64-bit integers: lane l holds two values whose indices differ only in one bit (a: that
// bit 0, b: 1) and whose other six bits are l's -- values 2l and 2l + 1, or l and l + 64.
// The transform is one butterfly per index bit in any order, so both layouts work.
__device__ __forceinline__ void fwht64(int64_t& a, int64_t& b, int lane) {
    {
        const int64_t s = a + b, d = a - b;
        a = s;
        b = d;
    }
    fwht64_stage<1>(a, b, lane);
    fwht64_stage<2>(a, b, lane);
    fwht64_stage<4>(a, b, lane);
    fwht64_stage<8>(a, b, lane);
    fwht64_stage<16>(a, b, lane);
    fwht64_stage<32>(a, b, lane);
}

// The same transform in binary64 (values, not units): every binary16 value and every
// partial sum (a multiple of 2^-24 below 2^23 in magnitude, 47 significant bits) is
// exact in binary64, so each butterfly is one exact fused multiply-add by +-1 and the
// result's conversion to binary32 is RN32 of the exact sum
template <int M>
__device__ __forceinline__ double lane_xor_f64(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = lane_xor<M>((uint32_t)u, lane), hi = lane_xor<M>((uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, lo | (hi << 32));
}
template <int M>
__device__ __forceinline__ void fwht64d_stage(double& a, double& b, int lane) {
    const double pa = lane_xor_f64<M>(a, lane), pb = lane_xor_f64<M>(b, lane);
    const double sg = (lane & M) ? -1.0 : 1.0;  // the pair's second member takes partner - own
    a = __builtin_fma(sg, a, pa);
    b = __builtin_fma(sg, b, pb);
}
__device__ __forceinline__ void fwht64d(double& a, double& b, int lane) {
    {
        const double s = a + b, d = a - b;
        a = s;
        b = d;
    }
    fwht64d_stage<1>(a, b, lane);
    fwht64d_stage<2>(a, b, lane);
    fwht64d_stage<4>(a, b, lane);
    fwht64d_stage<8>(a, b, lane);
    fwht64d_stage<16>(a, b, lane);
    fwht64d_stage<32>(a, b, lane);
}
// the lane's two rotated sums of two binary16 values (signs: nonzero -> negate), RN32
__device__ __forceinline__ void rotated_pair_f32(uint32_t x0, uint32_t x1, uint32_t sg0, uint32_t sg1, int lane,
                                                 float& r0, float& r1) {
    double a = (double)h2f(x0), b = (double)h2f(x1);
    if (sg0) a = -a;
    if (sg1) b = -b;
    fwht64d(a, b, lane);
    r0 = (float)a;
    r1 = (float)b;
}

// RN32 of the exact sum (units of 2^-24): a correctly rounded 64-bit integer
// conversion, then an exact power-of-two scaling (results are normal)
__device__ __forceinline__ float units_to_f32(int64_t u) { return __builtin_amdgcn_ldexpf(__ll2float_rn(u), -24); }

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
//
// window > 0 (the fp16 recent window): ring_k / ring_v hold the newest `window`
// tokens of every (sequence, KV head) at rows [s][h][t mod window][128] (strides
// stride_seq / stride_head); the packed cache holds the first seq_len[s] - window
// tokens and attention over the packed part reads only those.  k / v then point at
// the ring: in a step the token leaving the window (ring row (seq_len[s] - 1) mod
// window) is packed into slot seq_len[s] - window - 1 by the wave that appends, which
// then writes the step's new token (k_new / v_new rows, null: no step) to that ring
// row.  The same launch computes the window's attention as one more chunk (the last,
// index n_split - 1), reading the new token from k_new; when nothing leaves the
// window (seq_len[s] <= window) that chunk's workgroup writes the new ring row.
struct AppendArgs {
    const uint16_t* k;
    const uint16_t* v;
    int64_t stride_seq;
    int64_t stride_head;
    int32_t window;
    uint16_t* ring_k;
    uint16_t* ring_v;
    const uint16_t* k_new;
    const uint16_t* v_new;
    int64_t new_stride_seq;
    int64_t new_stride_head;
    // the rotated variant's fused step (matrix-core kernel only): queries rotated with
    // the key signs, the new token rotated and coded as the rotated quantizer codes it
    // (values too when v_signs != nullptr); nullptr: no rotation
    const uint8_t* k_signs;
    const uint8_t* v_signs;
};

// window token i of sequence s (position len - nw + i; ring row (r0 + i) mod window with
// r0 = (len - nw) mod window; the newest from k_new in a step)
__device__ __forceinline__ const uint16_t* window_row(const AppendArgs& a, const uint16_t* ring, const uint16_t* nw_row,
                                                      int s, int kvh, int i, int nw, int r0) {
    if (nw_row != nullptr && i == nw - 1) return nw_row + (int64_t)s * a.new_stride_seq + (int64_t)kvh * a.new_stride_head;
    int r = r0 + i;
    if (r >= a.window) r -= a.window;
    return ring + (int64_t)s * a.stride_seq + (int64_t)kvh * a.stride_head + (int64_t)r * kHeadDim;
}

// The window's chunks: window tokens (positions [len - nw, len), nw = min(len, window),
// at their binary16 values) are split into groups of kWindowChunk, each attended by
// one workgroup as one more split partial in the decode partials' format (m in log2
// units, l, unnormalised o) -- the last window_chunks(window) partials of the row.
constexpr int kWindowChunk = 32;
__host__ __device__ inline int window_chunks(int window) { return (window + kWindowChunk - 1) / kWindowChunk; }

// Window chunk wc of (s, kvh) for the g query heads: 256 threads, g <= GMAX <= 16;
// scratch: LDS of at least (g * 128 + 2 * g * 32) floats.
template <int GMAX>
__device__ __forceinline__ void window_chunk(const AppendArgs& a, const uint16_t* __restrict__ q, int n_q, int g,
                                             int s, int kvh, const int32_t* __restrict__ seq_len, float scale_log2,
                                             float* __restrict__ ws, int n_split, int wc, float* scratch) {
    const int tid = threadIdx.x;
    const int64_t len = seq_len[s] > 0 ? (int64_t)seq_len[s] : 0;
    const int nw = (int)(len < a.window ? len : a.window);
    const int r0 = (int)((len - nw) % a.window);
    const int base = wc * kWindowChunk;
    const int nc = nw - base < kWindowChunk ? (nw - base > 0 ? nw - base : 0) : kWindowChunk;
    float* s_q = scratch;                 // [g][128]
    float* s_p = scratch + g * kHeadDim;  // [g][32]: logits, then weights
    float* s_o = s_p + g * kWindowChunk;  // [g][32]: unused rows pad the odd tokens' share below
    for (int i = tid; i < g * kHeadDim; i += 256) s_q[i] = h2f(q[((int64_t)s * n_q + (int64_t)kvh * g) * kHeadDim + i]);
    __syncthreads();
    if (nc > 0) {  // logits: token i = tid / 8, coordinates 16j .. 16j + 15
        const int i = tid >> 3, j = tid & 7;
        const int ii = i < nc ? i : nc - 1;  // a valid row for every load
        const uint4* kr = (const uint4*)(window_row(a, a.ring_k, a.k_new, s, kvh, base + ii, nw, r0) + 16 * j);
        const uint4 k0 = kr[0], k1 = kr[1];
        const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        float kf[16];
#pragma unroll
        for (int e = 0; e < 8; ++e) { kf[2 * e] = h2f(kw[e] & 0xffffu); kf[2 * e + 1] = h2f(kw[e] >> 16); }
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            if (h < g) {
                const float* qh = s_q + h * kHeadDim + 16 * j;
                float z = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) z += qh[e] * kf[e];
                z += __shfl_xor(z, 1);
                z += __shfl_xor(z, 2);
                z += __shfl_xor(z, 4);
                if (j == 0 && i < nc) s_p[h * kWindowChunk + i] = z * scale_log2;
            }
        }
    }
    __syncthreads();
    // per head (32 lanes, one token each): max, weights, their sum
    float mh = -INFINITY, lh = 0.f;
    {
        const int h = tid >> 5, l = tid & 31;
        if (h < g && nc > 0) {
            float z = l < nc ? s_p[h * kWindowChunk + l] : -INFINITY;
            float mx = z;
            for (int off = 16; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
            const float pw = l < nc ? exp2f(z - mx) : 0.f;
            float ps = pw;
            for (int off = 16; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
            if (l < nc) s_p[h * kWindowChunk + l] = pw;
            mh = mx;
            lh = ps;
        }
    }
    __syncthreads();
    // output: thread (c, hh) takes coordinate c of every head over the tokens of parity hh
    const int c = tid & (kHeadDim - 1), hh = tid >> 7;
    float oacc[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) oacc[h] = 0.f;
    if (nc > 0) {
        uint32_t vr[kWindowChunk / 2];
#pragma unroll
        for (int u = 0; u < kWindowChunk / 2; ++u) {
            const int i = min(hh + 2 * u, nc - 1);
            vr[u] = window_row(a, a.ring_v, a.v_new, s, kvh, base + i, nw, r0)[c];
        }
#pragma unroll
        for (int u = 0; u < kWindowChunk / 2; ++u) {
            const int i = hh + 2 * u;
            if (i < nc) {
                const float vv = h2f(vr[u]);
#pragma unroll
                for (int h = 0; h < GMAX; ++h)
                    if (h < g) oacc[h] += s_p[h * kWindowChunk + i] * vv;
            }
        }
    }
    // the odd tokens' share into LDS (over s_q, no longer read), then the even lanes write
    __syncthreads();
    if (hh == 1) {
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
            if (h < g) s_q[h * kHeadDim + c] = oacc[h];
    }
    if ((tid & 31) == 0 && (tid >> 5) < g) { s_o[2 * (tid >> 5)] = mh; s_o[2 * (tid >> 5) + 1] = lh; }
    __syncthreads();
    constexpr int D2 = kHeadDim + 2;
    const int split = n_split - window_chunks(a.window) + wc;
    if (hh == 0) {
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            if (h < g) {
                float* part = ws + (((int64_t)s * n_q + (int64_t)kvh * g + h) * n_split + split) * D2;
                part[2 + c] = oacc[h] + s_q[h * kHeadDim + c];
                if (c == 0) { part[0] = s_o[2 * h]; part[1] = s_o[2 * h + 1]; }
            }
        }
    }
    // a step in which nothing leaves the window: the new token's ring row is free
    if (wc == 0 && a.k_new != nullptr && len >= 1 && len <= a.window && tid < kHeadDim) {
        const bool isv = tid >= kHeadDim / 2;
        const int e = tid & (kHeadDim / 2 - 1);
        const uint16_t* src = (isv ? a.v_new : a.k_new) + (int64_t)s * a.new_stride_seq + (int64_t)kvh * a.new_stride_head;
        uint16_t* dst = (isv ? a.ring_v : a.ring_k) + (int64_t)s * a.stride_seq + (int64_t)kvh * a.stride_head +
                        ((len - 1) % a.window) * kHeadDim;
        ((uint32_t*)dst)[e] = ((const uint32_t*)src)[e];
    }
}

struct DecodePlan {
    int kernel;           // KVQ_DECODE_GENERIC or KVQ_DECODE_MFMA
    int tiles_per_split;  // 64-token tiles per chunk
    int n_split;          // chunks per (sequence, KV head)
    int64_t workspace;    // bytes: the partials of n_split chunks, then table_bytes
    int64_t table_bytes;  // the generic kernel's query table (0 for the matrix-core kernel)
};
// workspace bytes of a plan whose launch carries n_chunks chunks (the window's included)
inline int64_t plan_workspace(const DecodePlan& p, int n_chunks) {
    return (p.workspace - p.table_bytes) / p.n_split * n_chunks + p.table_bytes;
}
// Returns 0 and fills the plan, or a negative kvq_status.
int plan_decode(const kvq_geom& g, int n_q_heads, int n_seq, int64_t max_len, int kernel, int tiles_per_split,
                DecodePlan* plan);
hipError_t launch_decode_partials(const kvq_geom& g, const DecodePlan& plan, int n_q_heads, const uint16_t* q,
                                  uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len,
                                  int n_seq, int64_t max_len, const uint8_t* k_bits, const float* k_sigma,
                                  const float* v_sigma, float softmax_scale, float* partials, hipStream_t st,
                                  const AppendArgs& app = AppendArgs{});
// one token per sequence into slot seq_len[s] - 1 (the decode step's append, alone)
// the vector-ALU kernel (kvq_decode_generic.hip): a query-table launch, then the
// chunks; the table lives after the partials of all n_chunks chunks
hipError_t launch_decode_generic(const kvq_geom& g, int tiles_per_split, int n_chunks, int n_q_heads,
                                 const uint16_t* q, uint8_t* cache, const int64_t* seq_byte_off,
                                 const int32_t* seq_len, int n_seq, int64_t max_len, const uint8_t* k_bits,
                                 const float* k_sigma, const float* v_sigma, float scale_log2, float* partials,
                                 hipStream_t st, const AppendArgs& app);
int64_t generic_table_bytes(const kvq_geom& g, int n_q_heads, int n_seq);
int generic_blocks_per_cu(const kvq_geom& g, int n_q_heads);
hipError_t launch_merge(int n_rows, int n_split, const float* partials, float* out, hipStream_t st);

// plain streaming read of `bytes` (a multiple of 16) by n_blocks workgroups; one word per
// workgroup to sink (kvq_decode.hip)
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, int n_blocks, hipStream_t st);

// the TurboQuant-MSE rotation variant (kvq_rotate.hip)
hipError_t launch_rot_quantize(const kvq_geom& g, const uint16_t* k, const uint16_t* v, int64_t stride_tok,
                               int64_t stride_head, int n_seq, const int64_t* first_slot, const int32_t* n_new,
                               const int64_t* src_row0, int max_new, const uint8_t* k_signs, const uint8_t* v_signs,
                               const float* v_sigma, uint8_t* cache, const int64_t* seq_byte_off, hipStream_t st);
hipError_t launch_rot_queries(const uint16_t* q, uint16_t* qr, const uint8_t* k_signs, int n_rows, int n_q, int g,
                              hipStream_t st);
hipError_t launch_rot_back(float* out, const uint8_t* v_signs, int n_rows, int n_q, int g, hipStream_t st);

// chunked prefill attention (kvq_prefill.hip)
struct PrefillPlan {
    int n_qb;           // query blocks (128 query rows each) per (sequence, KV head)
    int n_split;        // key-range splits per query block (1: the kernel writes the output itself)
    int64_t workspace;  // bytes of split partials (0 when n_split == 1)
};
int plan_prefill(const kvq_geom& g, int n_q_heads, int n_seq, int max_q, int64_t max_len, int n_split_req,
                 PrefillPlan* plan);
hipError_t launch_prefill(const kvq_geom& g, const PrefillPlan& plan, int n_q_heads, const uint16_t* q,
                          const uint8_t* cache, const int64_t* seq_byte_off, const int32_t* q_start,
                          const int32_t* n_q, int n_seq, int max_q, int64_t max_len, const uint8_t* k_bits,
                          const float* k_sigma, const float* v_sigma, float softmax_scale, float* out, float* ws,
                          hipStream_t st);


}  // namespace kvq
