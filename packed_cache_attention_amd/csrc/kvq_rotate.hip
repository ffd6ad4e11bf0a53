// kvq_rotate.hip -- the TurboQuant-MSE rotation variant: keys (and optionally values)
// rotated by a seeded random-sign Walsh-Hadamard transform before uniform scalar
// quantization, queries rotated once per step, outputs rotated back once per head.
// "RoPE-Aware Bit Allocation for KV-Cache Quantization" (abstract) builds Block-GTQ on
// TurboQuant-MSE; the related-papers page for "Quantization Dominates Rank Reduction
// for KV-Cache" names its key path "WHT + MSE".  This file is that baseline on the GPU.
//
// Rotation R = H diag(sg) / sqrt(128), H the Sylvester Hadamard matrix.  A binary16
// row x gives the exact sums S = H (sg * x) = sqrt(128) R x: every binary16 value is
// an integer count of 2^-24 below 2^40, so the sums are exact in 64-bit integers
// (|S| < 2^47) and in binary64; each is rounded once to binary32.  Codes compare S
// with the token norm times the Gaussian thresholds: code = #{j : S_i >= RN32(s * t_j)}
// (the normalised rotated coordinate S_i / s against the codebook of N(0, 1)).
//
// Queries and a decode step's new token give a row one wave: lane l holds coordinates
// 2l and 2l + 1, so the transform's first butterfly stage is lane-local and stage
// h = 2^k (k >= 1) pairs lane l with lane l ^ 2^(k-1) (the most lanes for these short,
// latency-bound launches).  The bulk quantizer and the output back-rotation give a row
// 16 lanes (below).
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {


// the lane's two rotated sums of a binary16 row (signs: 1 -> -1)
__device__ __forceinline__ void rotated_pair(uint32_t pair, const uint8_t* __restrict__ sg, int lane, float& s0,
                                             float& s1) {
    int64_t a = h2units(pair & 0xffffu), b = h2units(pair >> 16);
    if (sg[2 * lane]) a = -a;
    if (sg[2 * lane + 1]) b = -b;
    fwht64(a, b, lane);
    s0 = units_to_f32(a);
    s1 = units_to_f32(b);
}

// ---------------------------------------------------------------- 16 lanes per token
// The bulk quantizer gives each token 16 lanes of a row of the wave: lane j holds
// coordinates 8j .. 8j + 7.  Cross-lane steps pair lane j with j ^ 1, 2, 4, 8 inside
// the row of 16 through DPP: quad permutations for 1 and 2, a rotate by 8 for 8, and
// for 4 two rotates (by 12 for lanes 0-3 and 8-11, by 4 for lanes 4-7 and 12-15)
// selected by the DPP bank mask.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
template <int B>
__device__ __forceinline__ uint32_t row_xor(uint32_t x) {
    if (B == 0) return dpp_row<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    if (B == 1) return dpp_row<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    if (B == 3) return dpp_row<0x128>(x);  // row_ror:8
    const int t = __builtin_amdgcn_update_dpp(0, (int)x, 0x12C, 0xf, 0x5, false);  // row_ror:12, banks 0, 2
    return (uint32_t)__builtin_amdgcn_update_dpp(t, (int)x, 0x124, 0xf, 0xA, false);  // row_ror:4, banks 1, 3
}
template <int B>
__device__ __forceinline__ double row_xor64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = row_xor<B>((uint32_t)u), hi = row_xor<B>((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, lo | (hi << 32));
}
template <int B>
__device__ __forceinline__ float row_xorf(float v) {
    return __builtin_bit_cast(float, row_xor<B>(__builtin_bit_cast(uint32_t, v)));
}

// the token norm from the lane's eight binary16 values: the same balanced pairwise
// binary32 tree as token_norm (levels 1-3 inside the lane, 4-7 across lanes j ^ 1, 2,
// 4, 8; after level 5 a lane's four-lane group is uniform, so any lane of the other
// group completes level 6)
__device__ __forceinline__ float token_norm8(const uint32_t (&w)[4]) {
    float l1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = h2f(w[i] & 0xffffu), b = h2f(w[i] >> 16);
        l1[i] = a * a + b * b;  // both squares exact in binary32
    }
    float t = (l1[0] + l1[1]) + (l1[2] + l1[3]);
    t = t + row_xorf<0>(t);
    t = t + row_xorf<1>(t);
    t = t + row_xorf<2>(t);
    t = t + row_xorf<3>(t);
    return sqrtf(t);
}

// S = H (sg * x) over the token's 128 values, the lane's eight in a[]: exact in
// binary64 (each partial sum is a multiple of 2^-24 below 2^23, within 47 bits)
__device__ __forceinline__ void fwht128(double (&a)[8], int j) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!(i & h)) {
                const double u = a[i], v = a[i + h];
                a[i] = u + v;
                a[i + h] = u - v;
            }
    // lane bit b: the lane without it keeps u + v, the lane with it v' - u' (its own
    // value subtracted from its partner's), both exact: p + sgn * a
    const double s0 = (j & 1) ? -1.0 : 1.0, s1 = (j & 2) ? -1.0 : 1.0, s2 = (j & 4) ? -1.0 : 1.0,
                 s3 = (j & 8) ? -1.0 : 1.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_fma(s0, a[i], row_xor64<0>(a[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_fma(s1, a[i], row_xor64<1>(a[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_fma(s2, a[i], row_xor64<2>(a[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_fma(s3, a[i], row_xor64<3>(a[i]));
}

// binary16 values (sign bits flipped by neg) as binary64
__device__ __forceinline__ void halves_to_f64(const uint32_t (&w)[4], const uint32_t (&neg)[4], double (&a)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = w[i] ^ neg[i];
        a[2 * i] = (double)h2f(x & 0xffffu);
        a[2 * i + 1] = (double)h2f(x >> 16);
    }
}

// ---------------------------------------------------------------- quantize + pack
// One workgroup (4 waves) per (sequence, KV head, tile touched by the call).  Phase 1:
// each wave takes four tokens at a time, 16 lanes each (lane j: coordinates 8j ..
// 8j + 7): the token norm (the pairwise tree), the rotated sums and their codes,
// written to LDS code rows.  Phase 2: the tile's K records (every block at the same
// width, so field f of the K order is coordinate c_f = p(f/2) or q(f/2) at bit w*f),
// V runs and scales, one thread per word.
constexpr int kRotWaves = 4;
constexpr int kRotThreads = 64 * kRotWaves;

__global__ __launch_bounds__(kRotThreads) void rot_quantize_kernel(
    const uint16_t* __restrict__ kx, const uint16_t* __restrict__ vx, int64_t stride_tok, int64_t stride_head,
    const int64_t* __restrict__ first_slot, const int32_t* __restrict__ n_new, const int64_t* __restrict__ src_row0,
    int max_new, int64_t capacity, const uint8_t* __restrict__ k_signs, const uint8_t* __restrict__ v_signs,
    const float* __restrict__ v_sigma, uint8_t* __restrict__ cache, const int64_t* __restrict__ seq_byte_off,
    int pairing, int wk, int v_bits) {
    const int s = blockIdx.z, h = blockIdx.y;
    const int64_t first = first_slot[s];
    const int n = n_new[s];
    if (first < 0 || n <= 0 || n > max_new || first + n > capacity) return;
    const int64_t tau = first / kTile + blockIdx.x;
    const int64_t tile0 = tau * kTile;
    const int64_t lo_slot = max(first, tile0), hi_slot = min(first + (int64_t)n, tile0 + kTile);
    if (lo_slot >= hi_slot) return;
    const int lo_p = (int)(lo_slot - tile0), hi_p = (int)(hi_slot - tile0);
    const int k_budget = wk * kMaxBlocks;
    const int64_t SK = k_record_bytes(k_budget);
    const int64_t TB = tile_bytes(kHeadDim, k_budget, v_bits);
    const int RW = (int)(SK / 4), VW = 2 * v_bits;
    uint8_t* tile = cache + seq_byte_off[s] + ((int64_t)h * (capacity / kTile) + tau) * TB;

    __shared__ __attribute__((aligned(16))) uint8_t s_kc[kTile][kHeadDim + 8];  // codes [slot][coordinate]
    __shared__ __attribute__((aligned(16))) uint8_t s_vc[kTile][kHeadDim + 8];
    __shared__ float s_ks[kTile], s_vs[kTile];
    __shared__ float s_thr[512];
    __shared__ uint8_t s_ksg[kHeadDim], s_vsg[kHeadDim];
    __shared__ float s_vsig[kHeadDim];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool vrot = v_signs != nullptr;
    for (int i = tid; i < 510; i += kRotThreads) s_thr[i] = c_thresholds[i];
    if (tid < kHeadDim) {
        s_ksg[tid] = k_signs[h * kHeadDim + tid];
        s_vsg[tid] = vrot ? v_signs[h * kHeadDim + tid] : 0;
        const int blk = pairing == KVQ_PAIR_HALF ? (tid & (kMaxBlocks - 1)) : (tid >> 1);
        s_vsig[tid] = vrot ? 1.f : v_sigma[h * kMaxBlocks + blk];
    }
    for (int i = tid; i < kTile * (kHeadDim + 8) / 4; i += kRotThreads) {
        ((uint32_t*)s_kc)[i] = 0u;
        ((uint32_t*)s_vc)[i] = 0u;
    }
    __syncthreads();

    // ---- phase 1: norms, rotated sums, codes; four tokens per wave at a time (lanes
    // 16q .. 16q + 15 take token q of the four), every row requested before the first
    // is used
    const int j = lane & 15, tq = lane >> 4;
    uint32_t kneg[4], vneg[4];  // binary16 sign bits of the lane's coordinates' signs
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kneg[i] = (s_ksg[8 * j + 2 * i] ? 0x8000u : 0u) | (s_ksg[8 * j + 2 * i + 1] ? 0x80000000u : 0u);
        vneg[i] = (s_vsg[8 * j + 2 * i] ? 0x8000u : 0u) | (s_vsg[8 * j + 2 * i + 1] ? 0x80000000u : 0u);
    }
    constexpr int kRounds = kTile / (4 * kRotWaves);
    const int64_t row0 = src_row0[s] + (tile0 - first);
    uint32_t kw[kRounds][4], vw[kRounds][4];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        const int p = lo_p + 4 * (kRounds * wave + r) + tq;
        const int64_t rr = row0 + min(p, hi_p - 1);  // a valid row for every load
        const uint32_t* kr = (const uint32_t*)(kx + rr * stride_tok + (int64_t)h * stride_head + 8 * j);
        const uint32_t* vr = (const uint32_t*)(vx + rr * stride_tok + (int64_t)h * stride_head + 8 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kw[r][i] = kr[i];
            vw[r][i] = vr[i];
        }
    }
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        const int p0 = lo_p + 4 * (kRounds * wave + r);
        if (p0 >= hi_p) break;
        const int p = p0 + tq;
        const float sk = token_norm8(kw[r]), sv = token_norm8(vw[r]);
        double a[8];
        halves_to_f64(kw[r], kneg, a);
        fwht128(a, j);
        uint32_t kc[2] = {0u, 0u}, vc[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) kc[i >> 2] |= code_of(s_thr, (float)a[i], wk, 1.f, sk) << (8 * (i & 3));
        if (vrot) {
            halves_to_f64(vw[r], vneg, a);
            fwht128(a, j);
#pragma unroll
            for (int i = 0; i < 8; ++i) vc[i >> 2] |= code_of(s_thr, (float)a[i], v_bits, 1.f, sv) << (8 * (i & 3));
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t x = (vw[r][i >> 1] >> (16 * (i & 1))) & 0xffffu;
                vc[i >> 2] |= code_of(s_thr, h2f(x), v_bits, s_vsig[8 * j + i], sv) << (8 * (i & 3));
            }
        }
        if (p < hi_p) {
            *(uint2*)&s_kc[p][8 * j] = uint2{kc[0], kc[1]};
            *(uint2*)&s_vc[p][8 * j] = uint2{vc[0], vc[1]};
            if (j == 0) {
                s_ks[p] = sk;
                s_vs[p] = sv;
            }
        }
    }
    __syncthreads();

    // ---- phase 2: K records of the call's slots (field f = block f/2's p or q coordinate)
    const bool whole = lo_p == 0 && hi_p == kTile;
    for (int idx = tid; idx < kTile * RW; idx += kRotThreads) {
        const int p = idx / RW, k = idx - p * RW;
        if (p < lo_p || p >= hi_p) continue;
        uint32_t val = 0u;
        const int f_lo = (32 * k) / wk, f_hi = min(2 * kMaxBlocks - 1, (32 * k + 31) / wk);
        for (int f = f_lo; f <= f_hi; ++f) {
            const int b = f >> 1;
            const int c = pairing == KVQ_PAIR_HALF ? b + (f & 1) * kMaxBlocks : 2 * b + (f & 1);
            const int off = wk * f - 32 * k;
            const uint32_t code = s_kc[p][c];
            val |= off >= 0 ? code << off : code >> -off;
        }
        ((uint32_t*)tile)[p * RW + k] = val;
    }
    // V runs: word k of run c holds slots with bits in [32k, 32k + 32)
    uint32_t* vrun = (uint32_t*)(tile + kTile * SK);
    for (int idx = tid; idx < kHeadDim * VW; idx += kRotThreads) {
        const int c = idx & (kHeadDim - 1), k = idx >> 7;
        const int plo = 32 * k / v_bits, phi = min(kTile - 1, (32 * k + 31) / v_bits);
        uint32_t val = 0u;
        for (int p = plo; p <= phi; ++p) {
            if (p < lo_p || p >= hi_p) continue;
            const int off = p * v_bits - 32 * k;
            const uint32_t code = s_vc[p][c];
            val |= off >= 0 ? code << off : code >> -off;
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

// ---------------------------------------------------------------- queries, outputs
// row r of n_rows: query head r % n_q (KV head (r % n_q) / g); one wave per row.
__global__ __launch_bounds__(256) void rot_query_kernel(const uint16_t* __restrict__ q, uint16_t* __restrict__ qr,
                                                        const uint8_t* __restrict__ k_signs, int n_rows, int n_q,
                                                        int g) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= n_rows) return;
    const int kvh = (r % n_q) / g;
    const uint32_t pair = *(const uint32_t*)(q + (int64_t)r * kHeadDim + 2 * lane);
    float s0, s1;
    rotated_pair(pair, k_signs + kvh * kHeadDim, lane, s0, s1);
    const _Float16 a = (_Float16)(s0 * kRotSigma), b = (_Float16)(s1 * kRotSigma);
    *(uint32_t*)(qr + (int64_t)r * kHeadDim + 2 * lane) =
        (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// The same transform on binary32 values, the lane's eight in a[] (the output rotated
// back: rounding here is ordinary floating point, within the attention tolerance)
__device__ __forceinline__ void fwht128f(float (&a)[8], int j) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!(i & h)) {
                const float u = a[i], v = a[i + h];
                a[i] = u + v;
                a[i + h] = u - v;
            }
    const float s0 = (j & 1) ? -1.f : 1.f, s1 = (j & 2) ? -1.f : 1.f, s2 = (j & 4) ? -1.f : 1.f,
                s3 = (j & 8) ? -1.f : 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_fmaf(s0, a[i], row_xorf<0>(a[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_fmaf(s1, a[i], row_xorf<1>(a[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_fmaf(s2, a[i], row_xorf<2>(a[i]));
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_fmaf(s3, a[i], row_xorf<3>(a[i]));
}

// out row r <- diag(sg) H out_r / sqrt(128), in place: 16 lanes per row (lane j:
// coordinates 8j .. 8j + 7), 16 rows per workgroup; a row's lanes exit together, so
// the DPP exchanges of the rows left stay within live lanes
__global__ __launch_bounds__(256) void rot_back_kernel(float* __restrict__ out, const uint8_t* __restrict__ v_signs,
                                                       int n_rows, int n_q, int g) {
    const int j = threadIdx.x & 15;
    const int r = blockIdx.x * 16 + (threadIdx.x >> 4);
    if (r >= n_rows) return;
    const int kvh = (r % n_q) / g;
    float2* row = (float2*)(out + (int64_t)r * kHeadDim + 8 * j);
    float a[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float2 y = row[i];
        a[2 * i] = y.x;
        a[2 * i + 1] = y.y;
    }
    fwht128f(a, j);
    const uint8_t* sg = v_signs + kvh * kHeadDim + 8 * j;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x = a[i] * kRotSigma;
        a[i] = sg[i] ? -x : x;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) row[i] = float2{a[2 * i], a[2 * i + 1]};
}

// ---------------------------------------------------------------- decode-step preparation
// One launch for a rotated decode step: block (x < n_kv, s) packs sequence s's new
// token for KV head x at slot seq_len[s] - 1 (one wave: lane l owns coordinates 2l,
// 2l + 1; the same norms, rotated sums and codes as rot_quantize_kernel, the record
// OR-assembled in LDS and stored whole, the V codes OR-ed into their runs -- the slot's
// bits are zero in a zero-initialised cache); block (x = n_kv + r, s) rotates query
// head r of sequence s with its KV head's key signs.
__global__ __launch_bounds__(64) void rot_step_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ qr, const uint16_t* __restrict__ kx,
    const uint16_t* __restrict__ vx, int64_t stride_seq, int64_t stride_head, uint8_t* __restrict__ cache,
    const int64_t* __restrict__ seq_byte_off, const int32_t* __restrict__ seq_len, int64_t capacity,
    const uint8_t* __restrict__ k_signs, const uint8_t* __restrict__ v_signs, const float* __restrict__ v_sigma,
    int n_kv, int n_q, int g, int pairing, int wk, int v_bits) {
    const int s = blockIdx.y, x = blockIdx.x, lane = threadIdx.x;
    if (x >= n_kv) {  // a query row
        const int hq = x - n_kv;
        const int64_t r = (int64_t)s * n_q + hq;
        const uint32_t pair = *(const uint32_t*)(q + r * kHeadDim + 2 * lane);
        float s0, s1;
        rotated_pair(pair, k_signs + (hq / g) * kHeadDim, lane, s0, s1);
        const _Float16 a = (_Float16)(s0 * kRotSigma), b = (_Float16)(s1 * kRotSigma);
        *(uint32_t*)(qr + r * kHeadDim + 2 * lane) =
            (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
        return;
    }
    const int h = x;
    const int64_t slot = (int64_t)seq_len[s] - 1;
    if (slot < 0 || slot >= capacity) return;
    const int64_t tau = slot / kTile;
    const int p = (int)(slot - tau * kTile);
    const int k_budget = wk * kMaxBlocks;
    const int64_t SK = k_record_bytes(k_budget);
    const int64_t TB = tile_bytes(kHeadDim, k_budget, v_bits);
    uint8_t* tile = cache + seq_byte_off[s] + ((int64_t)h * (capacity / kTile) + tau) * TB;
    __shared__ float s_thr[510];
    __shared__ uint32_t s_rec[32];  // the slot's K record (at most 8 bits x 128 fields)
    const bool vrot = v_signs != nullptr;
    const int c0 = 2 * lane, c1 = 2 * lane + 1;
    const uint32_t kp = *(const uint32_t*)(kx + (int64_t)s * stride_seq + (int64_t)h * stride_head + c0);
    const uint32_t vp = *(const uint32_t*)(vx + (int64_t)s * stride_seq + (int64_t)h * stride_head + c0);
    float vs0 = 1.f, vs1 = 1.f;
    if (!vrot) {
        const int b0 = pairing == KVQ_PAIR_HALF ? (c0 & (kMaxBlocks - 1)) : (c0 >> 1);
        const int b1 = pairing == KVQ_PAIR_HALF ? (c1 & (kMaxBlocks - 1)) : (c1 >> 1);
        vs0 = v_sigma[h * kMaxBlocks + b0];
        vs1 = v_sigma[h * kMaxBlocks + b1];
    }
    for (int i = lane; i < 510; i += 64) s_thr[i] = c_thresholds[i];
    if (lane < 32) s_rec[lane] = 0u;
    const float sk = token_norm(kp), sv = token_norm(vp);
    float k0, k1, v0, v1;
    rotated_pair(kp, k_signs + h * kHeadDim, lane, k0, k1);
    if (vrot) {
        rotated_pair(vp, v_signs + h * kHeadDim, lane, v0, v1);
    } else {
        v0 = h2f(vp & 0xffffu);
        v1 = h2f(vp >> 16);
    }
    __syncthreads();
    const uint32_t kc[2] = {code_of(s_thr, k0, wk, 1.f, sk), code_of(s_thr, k1, wk, 1.f, sk)};
    const uint32_t vc[2] = {code_of(s_thr, v0, v_bits, vs0, sv), code_of(s_thr, v1, v_bits, vs1, sv)};
    // K record: every block has width wk, so field f = 2b + e (block b's first or second
    // coordinate) sits at bit wk * f
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int c = e ? c1 : c0;
        const int f = pairing == KVQ_PAIR_HALF ? 2 * (c & (kMaxBlocks - 1)) + (c >> 6) : c;
        const int off = wk * f, k = off >> 5, sh = off & 31;
        atomicOr(&s_rec[k], kc[e] << sh);
        if (sh + wk > 32) atomicOr(&s_rec[k + 1], kc[e] >> (32 - sh));
    }
    __syncthreads();
    if (lane < (int)(SK / 4)) ((uint32_t*)(tile + (int64_t)p * SK))[lane] = s_rec[lane];
    uint32_t* vrun = (uint32_t*)(tile + kTile * SK);
    const int vb = p * v_bits, vk = vb >> 5, vsh = vb & 31;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        uint32_t* run = vrun + (e ? c1 : c0) * 2 * v_bits;
        if (vc[e] == 0) continue;
        atomicOr(run + vk, vc[e] << vsh);
        if (vsh + v_bits > 32 && (vc[e] >> (32 - vsh)) != 0) atomicOr(run + vk + 1, vc[e] >> (32 - vsh));
    }
    if (lane == 0) {
        float* scl = (float*)(tile + kTile * SK + kHeadDim * 8 * v_bits);
        scl[p] = sk;
        scl[kTile + p] = sv;
    }
}

hipError_t launch_rot_step(const kvq_geom& g, int n_q_heads, int n_seq, const uint16_t* q, uint16_t* qr,
                           const uint16_t* k_new, const uint16_t* v_new, int64_t stride_seq, int64_t stride_head,
                           uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len,
                           const uint8_t* k_signs, const uint8_t* v_signs, const float* v_sigma, hipStream_t st) {
    dim3 grid(g.n_kv_heads + n_q_heads, n_seq);
    hipLaunchKernelGGL(rot_step_kernel, grid, dim3(64), 0, st, q, qr, k_new, v_new, stride_seq, stride_head, cache,
                       seq_byte_off, seq_len, g.capacity_tokens, k_signs, v_signs, v_sigma, g.n_kv_heads, n_q_heads,
                       n_q_heads / g.n_kv_heads, g.rope_pairing, g.k_budget / kMaxBlocks, g.v_bits);
    return hipGetLastError();
}

hipError_t launch_rot_quantize(const kvq_geom& g, const uint16_t* k, const uint16_t* v, int64_t stride_tok,
                               int64_t stride_head, int n_seq, const int64_t* first_slot, const int32_t* n_new,
                               const int64_t* src_row0, int max_new, const uint8_t* k_signs, const uint8_t* v_signs,
                               const float* v_sigma, uint8_t* cache, const int64_t* seq_byte_off, hipStream_t st) {
    const int max_tiles = (max_new + kTile - 1) / kTile + 1;  // a range may straddle one more tile
    dim3 grid(max_tiles, g.n_kv_heads, n_seq);
    hipLaunchKernelGGL(rot_quantize_kernel, grid, dim3(kRotThreads), 0, st, k, v, stride_tok, stride_head, first_slot,
                       n_new, src_row0, max_new, g.capacity_tokens, k_signs, v_signs, v_sigma, cache, seq_byte_off,
                       g.rope_pairing, g.k_budget / kMaxBlocks, g.v_bits);
    return hipGetLastError();
}

hipError_t launch_rot_queries(const uint16_t* q, uint16_t* qr, const uint8_t* k_signs, int n_rows, int n_q, int g,
                              hipStream_t st) {
    hipLaunchKernelGGL(rot_query_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, st, q, qr, k_signs, n_rows, n_q, g);
    return hipGetLastError();
}

hipError_t launch_rot_back(float* out, const uint8_t* v_signs, int n_rows, int n_q, int g, hipStream_t st) {
    hipLaunchKernelGGL(rot_back_kernel, dim3((n_rows + 15) / 16), dim3(256), 0, st, out, v_signs, n_rows, n_q, g);
    return hipGetLastError();
}

}  // namespace kvq
