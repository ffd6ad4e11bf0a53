// kvq_decode_mfma.h -- packed-cache GQA decode attention on the CDNA4 matrix
// cores (gfx950), for the packed-cache serving path of "RoPE-Aware Bit
// Allocation for KV-Cache Quantization" (abstract).
//
// Per 64-slot tile, one wave computes
//   z_t = s_t * sum_c (q_c sigma_c scale log2e) level[code_{t,c}]      (QK)
//   o  += sum_t p_t s^V_t level[vcode_{t,c}]   (times sigma^V_c at the end)  (PV)
// with the levels (exact binary16) as matrix operands and the fp32 factors
// q.sigma and p.s^V split into binary16 hi + lo parts, so the products keep
// about 22 bits.
//
// QK uses v_mfma_f32_32x32x16_f16 with a block-diagonal B operand: lane l decodes
// one token (slot sigma(l)), and all 64 lanes decode the SAME 8 K-order
// coordinates per instruction (K widths are per (layer, head), so field offsets
// and widths are wave-uniform).  Lanes 0-31 feed token set 0 into k-slots 0-7 and
// lanes 32-63 feed token set 1 into k-slots 8-15; B columns 0-15 read only k-slots
// 0-7 and columns 16-31 only k-slots 8-15, each column being (hi|lo, head).  The
// 32x32 accumulator then holds, in lane l, 16 logits of column l%32 for slots
// 16*(l/16) + i, i = 0..15 -- exactly the A-operand layout of the PV product
// v_mfma_f32_16x16x32_f16 (row = l%16 = (hi|lo, head), k = 8*(l/16) + j), so
// softmax weights never leave registers.  The PV B operand of lane l is 16
// consecutive slots of one coordinate, i.e. one contiguous 16*v-bit piece of a V
// run.  Codes become binary16 levels through LDS tables: two codes per lookup
// (one dword = two levels) for widths <= 4, one code per lookup for widths 5..8.
#include <math.h>

#pragma once
#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kMaxUnits = 24;          // 128 coordinates in 8-wide units, plus one partial unit per class
constexpr int kWaves = 4;
constexpr float kPrescale = 256.f;     // keeps q.sigma well inside the binary16 range

// pair tables (widths 1..4): entry a | b << w -> half2(level_w[a], level_w[b])
__host__ __device__ constexpr int pair_off(int w) { return w == 1 ? 0 : w == 2 ? 4 : w == 3 ? 20 : 84; }
constexpr int kPairEntries = 340;
// single tables (widths 5..8)
__host__ __device__ constexpr int single_off(int w) { return w == 5 ? 0 : w == 6 ? 32 : w == 7 ? 96 : 224; }
constexpr int kSingleEntries = 480;

union H8 {
    half8 h;
    uint32_t u[4];
    uint16_t s[8];
};

__device__ __forceinline__ uint32_t alignbit(uint32_t hi, uint32_t lo, uint32_t s) {
    return __builtin_amdgcn_alignbit(hi, lo, s);
}

// bits [r, r + n) (n <= 16) of the 64-bit value hi:lo
__device__ __forceinline__ uint32_t field64(uint32_t lo, uint32_t hi, int r, int n) {
    const uint32_t x = r >= 32 ? (hi >> (r - 32)) : alignbit(hi, lo, (uint32_t)r);
    return x & ((1u << n) - 1u);
}

struct MfmaSmem {
    uint32_t pair[kPairEntries];
    uint16_t single[kSingleEntries];
    // binary16 hi/lo of q.sigma.scale by padded position: width class w occupies whole
    // 8-position units (its last unit zero-padded), classes in descending width
    alignas(16) uint16_t qsplit[2][8][8 * kMaxUnits];
    alignas(16) uint16_t qzero[8];                // zero operand for the off-diagonal B lanes
    int cls_start[9], cls_units[9], cls_ubase[9]; // per width class: record bit offset, units, first unit
    float vsig[kHeadDim];
    alignas(16) float alpha[kWaves][8];
    float wm[kWaves][8], wl[kWaves][8];
    float wo[kWaves][8][kHeadDim];
    int nf;
};

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

// Two equal-width fields at compile-time bit offset REL of the 64-bit window hi:lo,
// returned as two binary16 levels in one dword.
template <int W, int REL>
__device__ __forceinline__ uint32_t decode_pair(const MfmaSmem& sm, uint32_t lo, uint32_t hi) {
    uint32_t x;
    if (REL >= 32) x = hi >> (REL - 32);
    else if (REL + 2 * W <= 32) x = lo >> REL;
    else x = alignbit(hi, lo, REL);
    if (W <= 4) return sm.pair[pair_off(W) + (x & ((1u << (2 * W)) - 1u))];
    constexpr uint32_t m = (1u << W) - 1u;
    return (uint32_t)sm.single[single_off(W) + (x & m)] | ((uint32_t)sm.single[single_off(W) + ((x >> W) & m)] << 16);
}

// QK over the units of one width class: window of 8 fields -> A operand, q split -> B
template <int W, int RD>
__device__ __forceinline__ void qk_class(const MfmaSmem& sm, const uint32_t (&rec)[RD + 2], int start, int units,
                                         int ubase, const uint16_t* qb_src, bool bdiag, floatx16& acc) {
    for (int j = 0; j < units; ++j) {
        const int st = start + j * 8 * W;
        const int d = min(st >> 5, RD > 0 ? RD - 1 : 0);
        const uint32_t sh = (uint32_t)(st & 31);
        const uint32_t d0 = rec[d], d1 = rec[d + 1], d2 = rec[d + 2];
        const uint32_t lo = alignbit(d1, d0, sh), hi = alignbit(d2, d1, sh);
        H8 a;
        a.u[0] = decode_pair<W, 0>(sm, lo, hi);
        a.u[1] = decode_pair<W, 2 * W>(sm, lo, hi);
        a.u[2] = decode_pair<W, 4 * W>(sm, lo, hi);
        a.u[3] = decode_pair<W, 6 * W>(sm, lo, hi);
        H8 b;
        const uint4 q4 = *(const uint4*)(bdiag ? qb_src + 8 * (ubase + j) : sm.qzero);
        b.u[0] = q4.x; b.u[1] = q4.y; b.u[2] = q4.z; b.u[3] = q4.w;
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.h, b.h, acc, 0, 0, 0);
    }
}

template <int V, int RD>
__global__ __launch_bounds__(256) void decode_mfma_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, const int64_t* __restrict__ seq_byte_off,
    const int32_t* __restrict__ seq_len, int64_t max_len, int64_t capacity, const uint8_t* __restrict__ k_bits,
    const float* __restrict__ k_sigma, const float* __restrict__ v_sigma, float scale_log2, int n_q, int g,
    int pairing, int k_budget, int tiles_per_split, int n_split, float* __restrict__ ws) {
    __shared__ MfmaSmem sm;
    const int split = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t len = min(max((int64_t)seq_len[s], (int64_t)0), max_len);
    const int64_t n_tiles_seq = (len + kTile - 1) / kTile;
    const int64_t t0 = (int64_t)split * tiles_per_split;
    const int64_t t1 = min(t0 + tiles_per_split, n_tiles_seq);

    // ------------------------------------------------------------------ prologue
    for (int i = tid; i < kPairEntries; i += 256) {
        const int w = i < 4 ? 1 : i < 20 ? 2 : i < 84 ? 3 : 4;
        const int e = i - pair_off(w);
        const int a = e & ((1 << w) - 1), b = e >> w;
        sm.pair[i] = (uint32_t)c_levels[KVQ_CB_OFF(w) + a] | ((uint32_t)c_levels[KVQ_CB_OFF(w) + b] << 16);
    }
    for (int i = tid; i < kSingleEntries; i += 256) {
        const int w = i < 32 ? 5 : i < 96 ? 6 : i < 224 ? 7 : 8;
        sm.single[i] = c_levels[KVQ_CB_OFF(w) + i - single_off(w)];
    }
    for (int c = tid; c < kHeadDim; c += 256) {
        const int i = pairing == KVQ_PAIR_HALF ? (c & (kMaxBlocks - 1)) : (c >> 1);
        sm.vsig[c] = v_sigma[kvh * kMaxBlocks + i];
    }
    for (int i = tid; i < 2 * 8 * 8 * kMaxUnits; i += 256) (&sm.qsplit[0][0][0])[i] = 0;
    if (tid < 8) sm.qzero[tid] = 0;
    __syncthreads();
    if (wave == 0) {
        // width classes in descending order; a block's fields sit at its rank within its class
        const int i = lane;
        const int my_w = k_bits[kvh * kMaxBlocks + i];
        const float my_ksig = k_sigma[kvh * kMaxBlocks + i];
        const unsigned long long below = (1ull << i) - 1ull;
        int start = 0, ubase = 0, my_pos = 0;
#pragma unroll
        for (int w = 8; w >= 1; --w) {
            const unsigned long long mk = __ballot(my_w == w);
            const int nfw = 2 * __popcll(mk), units = (nfw + 7) >> 3;
            if (i == 0) { sm.cls_start[w] = start; sm.cls_units[w] = units; sm.cls_ubase[w] = ubase; }
            if (my_w == w) my_pos = 8 * ubase + 2 * __popcll(mk & below);
            start += nfw * w;
            ubase += units;
        }
        if (my_w > 0) {
            const int p = pairing == KVQ_PAIR_HALF ? i : 2 * i;
            const int qq = pairing == KVQ_PAIR_HALF ? i + kMaxBlocks : 2 * i + 1;
            for (int hh = 0; hh < g; ++hh) {
                const uint16_t* qrow = q + ((int64_t)s * n_q + kvh * g + hh) * kHeadDim;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float v = h2f(qrow[e ? qq : p]) * my_ksig * scale_log2 * kPrescale;
                    const _Float16 hi = (_Float16)v;
                    const _Float16 lo = (_Float16)(v - (float)hi);
                    sm.qsplit[0][hh][my_pos + e] = __builtin_bit_cast(uint16_t, hi);
                    sm.qsplit[1][hh][my_pos + e] = __builtin_bit_cast(uint16_t, lo);
                }
            }
        }
    }
    __syncthreads();
    int cstart[9], cunits[9], cubase[9];
#pragma unroll
    for (int w = 1; w <= 8; ++w) {
        cstart[w] = __builtin_amdgcn_readfirstlane(sm.cls_start[w]);
        cunits[w] = __builtin_amdgcn_readfirstlane(sm.cls_units[w]);
        cubase[w] = __builtin_amdgcn_readfirstlane(sm.cls_ubase[w]);
    }

    const int col = lane & 31;
    const bool bdiag = (col >> 4) == (lane >> 5);
    const uint16_t* qb_src = bdiag ? &sm.qsplit[(col >> 3) & 1][col & 7][0] : nullptr;
    // slot decoded by this lane for QK: token set lane/32, row m = lane%32
    const int m = lane & 31;
    const int qslot = 16 * (2 * ((m >> 2) & 1) + (lane >> 5)) + 4 * (m >> 3) + (m & 3);
    const int grp = lane >> 4;       // PV k group: slots 16*grp .. 16*grp+15
    const int row = lane & 15;       // PV row = (hi|lo) * 8 + head
    const bool lo_row = row >= 8;

    const int64_t SK = 4 * RD;
    const int64_t TB = tile_bytes(kHeadDim, k_budget, V);
    const uint8_t* head_base = cache + seq_byte_off[s] + (int64_t)kvh * (capacity / kTile) * TB;
    constexpr int NW = (16 * V + 31) / 32;  // words of one lane's V piece

    floatx4 o[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) o[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;

    // ------------------------------------------------------------------ tiles
    for (int64_t tau = t0 + wave; tau < t1; tau += kWaves) {
        const uint8_t* tile = head_base + tau * TB;
        const int nvalid = (int)min((int64_t)kTile, len - tau * kTile);
        const float* scl = (const float*)(tile + kTile * SK + kHeadDim * 8 * V);
        const uint8_t* vsec = tile + kTile * SK;
        // ---- issue every load of the tile first
        uint32_t rec[RD + 2];
#pragma unroll
        for (int k = 0; k < RD / 4; ++k) {
            const uint4 v4 = *(const uint4*)(tile + qslot * SK + 16 * k);
            rec[4 * k] = v4.x; rec[4 * k + 1] = v4.y; rec[4 * k + 2] = v4.z; rec[4 * k + 3] = v4.w;
        }
        rec[RD] = 0; rec[RD + 1] = 0;
        uint32_t vraw[8][NW + 1];
        uint32_t vsh[8];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const int byte0 = (16 * ct + row) * 8 * V + 2 * V * grp;
            const uint32_t* w = (const uint32_t*)(vsec + (byte0 & ~3));
            vsh[ct] = (uint32_t)(byte0 & 3) * 8;
#pragma unroll
            for (int k = 0; k <= NW; ++k) vraw[ct][k] = w[k];
        }
        float4 skv[4], svv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            skv[i] = *(const float4*)(scl + 16 * grp + 4 * i);
            svv[i] = *(const float4*)(scl + kTile + 16 * grp + 4 * i);
        }
        // ---- QK: this lane's token, 8 fields of one width class per instruction
        floatx16 acc = {};
        qk_class<8, RD>(sm, rec, cstart[8], cunits[8], cubase[8], qb_src, bdiag, acc);
        qk_class<7, RD>(sm, rec, cstart[7], cunits[7], cubase[7], qb_src, bdiag, acc);
        qk_class<6, RD>(sm, rec, cstart[6], cunits[6], cubase[6], qb_src, bdiag, acc);
        qk_class<5, RD>(sm, rec, cstart[5], cunits[5], cubase[5], qb_src, bdiag, acc);
        qk_class<4, RD>(sm, rec, cstart[4], cunits[4], cubase[4], qb_src, bdiag, acc);
        qk_class<3, RD>(sm, rec, cstart[3], cunits[3], cubase[3], qb_src, bdiag, acc);
        qk_class<2, RD>(sm, rec, cstart[2], cunits[2], cubase[2], qb_src, bdiag, acc);
        qk_class<1, RD>(sm, rec, cstart[1], cunits[1], cubase[1], qb_src, bdiag, acc);
        // ---- logits: hi + lo columns (lane l and l^8), token scale, ragged-tail mask
        float z[16];
        const float sk[16] = {skv[0].x, skv[0].y, skv[0].z, skv[0].w, skv[1].x, skv[1].y, skv[1].z, skv[1].w,
                              skv[2].x, skv[2].y, skv[2].z, skv[2].w, skv[3].x, skv[3].y, skv[3].z, skv[3].w};
        const float sv[16] = {svv[0].x, svv[0].y, svv[0].z, svv[0].w, svv[1].x, svv[1].y, svv[1].z, svv[1].w,
                              svv[2].x, svv[2].y, svv[2].z, svv[2].w, svv[3].x, svv[3].y, svv[3].z, svv[3].w};
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = (acc[i] + dpp_ror8(acc[i])) * sk[i] * (1.f / kPrescale);
        if (nvalid < kTile) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (16 * grp + i >= nvalid) z[i] = -INFINITY;
        }
        // ---- online softmax: a head's 64 logits sit in the lanes with equal lane%16
        float tm = z[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) tm = fmaxf(tm, z[i]);
        tm = xor32_max(xor16_max(tm));
        const float mnew = fmaxf(mrun, tm);
        const float alpha = exp2f(mrun - mnew);
        mrun = mnew;
        float psum = 0.f;
        H8 pa[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = exp2f(z[i] - mnew);
            psum += p;
            const float pv = p * sv[i];
            const _Float16 ph = (_Float16)pv;
            const _Float16 pl = (_Float16)(pv - (float)ph);
            pa[i >> 3].s[i & 7] = __builtin_bit_cast(uint16_t, lo_row ? pl : ph);
        }
        lrun = lrun * alpha + psum;
        // rescale the PV accumulator rows (row 4*(lane/16) + j holds head (row & 7))
        if (__ballot(alpha != 1.f)) {
            if (lane < 8) sm.alpha[wave][lane] = alpha;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            const float4 al = *(const float4*)&sm.alpha[wave][4 * (grp & 1)];
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                o[ct][0] *= al.x; o[ct][1] *= al.y; o[ct][2] *= al.z; o[ct][3] *= al.w;
            }
            __builtin_amdgcn_wave_barrier();
        }
        // ---- PV: B operand = 16 consecutive slots of coordinate 16*ct + lane%16
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            uint32_t nw[NW + 1];
#pragma unroll
            for (int k = 0; k < NW; ++k) nw[k] = alignbit(vraw[ct][k + 1], vraw[ct][k], vsh[ct]);
            nw[NW] = 0;
            H8 b0, b1;
#pragma unroll
            for (int pr = 0; pr < 8; ++pr) {
                const int bit = 2 * V * pr;
                const int k = bit >> 5, r = bit & 31;
                uint32_t val;
                if (V <= 4) {
                    const uint32_t idx = (r + 2 * V <= 32) ? ((nw[k] >> r) & ((1u << (2 * V)) - 1u))
                                                          : (alignbit(nw[k + 1], nw[k], r) & ((1u << (2 * V)) - 1u));
                    val = sm.pair[pair_off(V) + idx];
                } else {
                    const int bit2 = bit + V, k2 = bit2 >> 5, r2 = bit2 & 31;
                    const uint32_t ca = (r + V <= 32) ? ((nw[k] >> r) & ((1u << V) - 1u))
                                                      : (alignbit(nw[k + 1], nw[k], r) & ((1u << V) - 1u));
                    const uint32_t cb = (r2 + V <= 32) ? ((nw[k2] >> r2) & ((1u << V) - 1u))
                                                       : (alignbit(nw[k2 + 1], nw[k2], r2) & ((1u << V) - 1u));
                    val = (uint32_t)sm.single[single_off(V) + ca] | ((uint32_t)sm.single[single_off(V) + cb] << 16);
                }
                if (pr < 4) b0.u[pr] = val; else b1.u[pr - 4] = val;
            }
            o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[0].h, b0.h, o[ct], 0, 0, 0);
            o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[1].h, b1.h, o[ct], 0, 0, 0);
        }
    }

    // ------------------------------------------------------------------ combine
    // l: sum over the four slot groups (lanes l, l^16, l^32, l^48) of a head's hi row
    const float lsum = xor32_sum(xor16_sum(lrun));
    // o: rows r (hi) and r+8 (lo) of the same head sit in lanes l and l^32
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[ct][j] = xor32_sum(o[ct][j]);
    if (lane < 8) { sm.wm[wave][lane] = mrun; sm.wl[wave][lane] = lsum; }
    if (lane < 32) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) sm.wo[wave][4 * (lane >> 4) + j][16 * ct + (lane & 15)] = o[ct][j];
    }
    __syncthreads();
    // merge the four waves and write this chunk's partials
    const int D2 = kHeadDim + 2;
    for (int idx = tid; idx < g * kHeadDim; idx += 256) {
        const int hh = idx >> 7, c = idx & 127;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.wm[w][hh]);
        float l = 0.f, acc = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float a = exp2f(sm.wm[w][hh] - M);
                l += a * sm.wl[w][hh];
                acc += a * sm.wo[w][hh][c];
            }
        }
        float* part = ws + (((int64_t)s * n_q + kvh * g + hh) * n_split + split) * D2;
        part[2 + c] = acc * sm.vsig[c];
        if (c == 0) { part[0] = M; part[1] = l; }
    }
}

// launch for one value width V (instantiated in kvq_decode_mfma_v<V>.hip)
template <int V>
hipError_t launch_mfma_v(const kvq_geom& g, const DecodePlan& plan, int n_q_heads, const uint16_t* q,
                         const uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len, int n_seq,
                         int64_t max_len, const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                         float scale_log2, float* partials, hipStream_t st) {
    const int grp = n_q_heads / g.n_kv_heads;
    const int rd = (int)(k_record_bytes(g.k_budget) / 4);
    dim3 grid(plan.n_split, g.n_kv_heads, n_seq);
#define KVQ_LAUNCH(RDV)                                                                                        \
    if (rd == RDV) {                                                                                            \
        hipLaunchKernelGGL((decode_mfma_kernel<V, RDV>), grid, dim3(256), 0, st, q, cache, seq_byte_off,       \
                           seq_len, max_len, g.capacity_tokens, k_bits, k_sigma, v_sigma, scale_log2, n_q_heads, \
                           grp, g.rope_pairing, g.k_budget, plan.tiles_per_split, plan.n_split, partials);      \
        return hipGetLastError();                                                                               \
    }
    KVQ_LAUNCH(0) KVQ_LAUNCH(4) KVQ_LAUNCH(8) KVQ_LAUNCH(12) KVQ_LAUNCH(16)
#undef KVQ_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace kvq
