// kvq_decode_mfma.hip -- packed-cache GQA decode attention on the CDNA4 matrix
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

#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kUnits = 16;             // 128 coordinates / 8 per QK instruction
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
    alignas(16) uint16_t qsplit[2][8][kHeadDim];  // [hi|lo][head][K-order position] binary16 of q.sigma.scale
    int unit_start[kUnits];                // bit offset of unit u in a K record
    uint32_t unit_pairs[kUnits][4];        // per pair: rel offset | width << 8 (width 0 = empty)
    float vsig[kHeadDim];
    alignas(16) float alpha[kWaves][8];
    float wm[kWaves][8], wl[kWaves][8];
    float wo[kWaves][8][kHeadDim];
    int nf;
};

template <int V>
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
    // level tables
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
    // K order from the block widths: rank by (width desc, block asc) with wave ballots
    int my_w = 0, my_rank = 0, my_off = 0;
    float my_ksig = 0.f;
    if (wave == 0) {
        const int i = lane;
        my_w = k_bits[kvh * kMaxBlocks + i];
        my_ksig = k_sigma[kvh * kMaxBlocks + i];
        const unsigned long long below = (1ull << i) - 1ull;
        int rank = 0, off = 0;
#pragma unroll
        for (int w = 8; w >= 1; --w) {
            const unsigned long long m = __ballot(my_w == w);
            if (w > my_w) { rank += __popcll(m); off += 2 * w * __popcll(m); }
            if (w == my_w) { rank += __popcll(m & below); off += 2 * w * __popcll(m & below); }
        }
        my_rank = rank;
        my_off = off;
        const int nf = 2 * __popcll(__ballot(my_w > 0));
        if (i == 0) sm.nf = nf;
    }
    for (int c = tid; c < kHeadDim; c += 256) {
        const int i = pairing == KVQ_PAIR_HALF ? (c & (kMaxBlocks - 1)) : (c >> 1);
        sm.vsig[c] = v_sigma[kvh * kMaxBlocks + i];
    }
    // q.sigma.scale split into binary16 hi + lo, stored by K-order position
    // (positions beyond the field count and heads beyond the group are zero)
    for (int i = tid; i < 2 * 8 * kHeadDim; i += 256) (&sm.qsplit[0][0][0])[i] = 0;
    __syncthreads();
    if (wave == 0 && my_w > 0) {
        const int i = lane;
        const int p = pairing == KVQ_PAIR_HALF ? i : 2 * i;
        const int qq = pairing == KVQ_PAIR_HALF ? i + kMaxBlocks : 2 * i + 1;
        for (int hh = 0; hh < g; ++hh) {
            const uint16_t* qrow = q + ((int64_t)s * n_q + kvh * g + hh) * kHeadDim;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int c = e ? qq : p;
                const float v = h2f(qrow[c]) * my_ksig * scale_log2 * kPrescale;
                const _Float16 hi = (_Float16)v;
                const _Float16 lo = (_Float16)(v - (float)hi);
                sm.qsplit[0][hh][2 * my_rank + e] = __builtin_bit_cast(uint16_t, hi);
                sm.qsplit[1][hh][2 * my_rank + e] = __builtin_bit_cast(uint16_t, lo);
            }
        }
    }
    // unit table: unit u = K-order positions 8u..8u+7, four pairs of equal width
    if (wave == 0 && my_w > 0) {
        const int pos = 2 * my_rank;  // this block's pair starts at an even position
        const int u = pos >> 3, pr = (pos & 7) >> 1;
        sm.unit_pairs[u][pr] = 0;     // filled below once the unit start is known
    }
    __syncthreads();
    const int nf = sm.nf;
    const int n_units = (nf + 7) >> 3;
    if (wave == 0 && my_w > 0) {
        const int pos = 2 * my_rank;
        const int u = pos >> 3, pr = (pos & 7) >> 1;
        if (pr == 0) sm.unit_start[u] = my_off;
    }
    __syncthreads();
    if (wave == 0 && my_w > 0) {
        const int pos = 2 * my_rank;
        const int u = pos >> 3, pr = (pos & 7) >> 1;
        sm.unit_pairs[u][pr] = (uint32_t)(my_off - sm.unit_start[u]) | ((uint32_t)my_w << 8);
    }
    if (tid < kUnits * 4) {
        const int u = tid >> 2, pr = tid & 3;
        if (8 * u + 2 * pr >= nf) sm.unit_pairs[u][pr] = 0;
    }
    __syncthreads();

    // per-lane operand registers: QK B operand (block-diagonal q split), one per unit
    const int col = lane & 31;
    const bool bdiag = (col >> 4) == (lane >> 5);
    const int qhead = col & 7, qhl = (col >> 3) & 1;
    half8 qb[kUnits];
#pragma unroll
    for (int u = 0; u < kUnits; ++u) {
        H8 t;
        if (bdiag && u < n_units) {
            const uint4 w4 = *(const uint4*)&sm.qsplit[qhl][qhead][8 * u];
            t.u[0] = w4.x; t.u[1] = w4.y; t.u[2] = w4.z; t.u[3] = w4.w;
        } else {
            t.u[0] = t.u[1] = t.u[2] = t.u[3] = 0;
        }
        qb[u] = t.h;
    }
    // slot this lane decodes for QK: token set (lane/32), row m = lane%32
    const int m = lane & 31;
    const int qslot = 16 * (2 * ((m >> 2) & 1) + (lane >> 5)) + 4 * (m >> 3) + (m & 3);
    const int grp = lane >> 4;       // PV k group: slots 16*grp .. 16*grp+15
    const int row = lane & 15;       // PV row = (hi|lo) * 8 + head
    const bool lo_row = row >= 8;

    const int64_t SK = k_record_bytes(k_budget);
    const int64_t TB = tile_bytes(kHeadDim, k_budget, V);
    const uint8_t* head_base = cache + seq_byte_off[s] + (int64_t)kvh * (capacity / kTile) * TB;

    floatx4 o[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) o[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.f;

    // ------------------------------------------------------------------ tiles
    for (int64_t tau = t0 + wave; tau < t1; tau += kWaves) {
        const uint8_t* tile = head_base + tau * TB;
        const int nvalid = (int)min((int64_t)kTile, len - tau * kTile);
        const float* scl = (const float*)(tile + kTile * SK + kHeadDim * 8 * V);
        // scales of the 16 slots this lane holds in the QK accumulator / PV operand
        float sk[16], sv[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 a = *(const float4*)(scl + 16 * grp + 4 * i);
            const float4 b = *(const float4*)(scl + kTile + 16 * grp + 4 * i);
            sk[4 * i] = a.x; sk[4 * i + 1] = a.y; sk[4 * i + 2] = a.z; sk[4 * i + 3] = a.w;
            sv[4 * i] = b.x; sv[4 * i + 1] = b.y; sv[4 * i + 2] = b.z; sv[4 * i + 3] = b.w;
        }
        // ---- QK: decode this lane's token, 8 coordinates per instruction
        floatx16 acc = {};
        const uint32_t* rec = (const uint32_t*)(tile + qslot * SK);
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            if (u < n_units) {
                const int st = sm.unit_start[u];
                const uint32_t* w = rec + (st >> 5);
                const uint32_t d0 = w[0], d1 = w[1], d2 = w[2];
                const uint32_t sh = (uint32_t)(st & 31);
                const uint32_t lo = alignbit(d1, d0, sh), hi = alignbit(d2, d1, sh);
                H8 a;
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const uint32_t meta = sm.unit_pairs[u][pr];
                    const int wd = (int)(meta >> 8), rel = (int)(meta & 0xff);
                    uint32_t val = 0;
                    if (wd >= 1 && wd <= 4) {
                        val = sm.pair[pair_off(wd) + field64(lo, hi, rel, 2 * wd)];
                    } else if (wd >= 5) {
                        const uint32_t ca = field64(lo, hi, rel, wd), cb = field64(lo, hi, rel + wd, wd);
                        val = (uint32_t)sm.single[single_off(wd) + ca] | ((uint32_t)sm.single[single_off(wd) + cb] << 16);
                    }
                    a.u[pr] = val;
                }
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.h, qb[u], acc, 0, 0, 0);
            }
        }
        // ---- logits: hi + lo columns (lanes l and l^8), token scale, mask
        float z[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float other = __shfl_xor(acc[i], 8);
            float v = (acc[i] + other) * sk[i] * (1.f / kPrescale);
            if (16 * grp + i >= nvalid) v = -INFINITY;
            z[i] = v;
        }
        // ---- online softmax: the head's 64 logits sit in lanes with equal lane%16
        float tm = z[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) tm = fmaxf(tm, z[i]);
        tm = fmaxf(tm, __shfl_xor(tm, 16));
        tm = fmaxf(tm, __shfl_xor(tm, 32));
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
        // rescale the PV accumulator rows (row = 4*(lane/16) + j holds head (row & 7))
        if (__ballot(alpha != 1.f)) {
            if (lane < 8) sm.alpha[wave][lane] = alpha;
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            const float4 al = *(const float4*)&sm.alpha[wave][4 * (grp & 1)];
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                o[ct][0] *= al.x; o[ct][1] *= al.y; o[ct][2] *= al.z; o[ct][3] *= al.w;
            }
            __builtin_amdgcn_wave_barrier();
        }
        // ---- PV: B operand = 16 consecutive slots of coordinate 16*ct + lane%16
        const uint8_t* vsec = tile + kTile * SK;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const int c = 16 * ct + row;
            const int byte0 = c * 8 * V + 2 * V * grp;
            const uint32_t* w = (const uint32_t*)(vsec + (byte0 & ~3));
            const uint32_t sh = (uint32_t)(byte0 & 3) * 8;
            constexpr int NW = (16 * V + 31) / 32;  // normalised words
            uint32_t raw[NW + 1], nw[NW + 1];
#pragma unroll
            for (int k = 0; k <= NW; ++k) raw[k] = w[k];
#pragma unroll
            for (int k = 0; k < NW; ++k) nw[k] = alignbit(raw[k + 1], raw[k], sh);
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
    // l: sum of the hi-row lanes of each head over the four slot groups
    float lsum = lrun;
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    // o: rows r (hi) and r+8 (lo) of the same head sit in lanes l and l^32
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[ct][j] += __shfl_xor(o[ct][j], 32);
    if (lane < 8) { sm.wm[wave][lane] = mrun; sm.wl[wave][lane] = lsum; }
    if (lane < 32) {
        // lane holds head rows 4*(lane/16) + j, column 16*ct + lane%16
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

hipError_t launch_decode_mfma(const kvq_geom& g, const DecodePlan& plan, int n_q_heads, const uint16_t* q,
                              const uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len, int n_seq,
                              int64_t max_len, const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                              float scale_log2, float* partials, hipStream_t st) {
    const int grp = n_q_heads / g.n_kv_heads;
    dim3 grid(plan.n_split, g.n_kv_heads, n_seq);
#define KVQ_LAUNCH(VB)                                                                                         \
    case VB:                                                                                                   \
        hipLaunchKernelGGL(decode_mfma_kernel<VB>, grid, dim3(256), 0, st, q, cache, seq_byte_off, seq_len,   \
                           max_len, g.capacity_tokens, k_bits, k_sigma, v_sigma, scale_log2, n_q_heads, grp,   \
                           g.rope_pairing, g.k_budget, plan.tiles_per_split, plan.n_split, partials);          \
        break;
    switch (g.v_bits) {
        KVQ_LAUNCH(1) KVQ_LAUNCH(2) KVQ_LAUNCH(3) KVQ_LAUNCH(4) KVQ_LAUNCH(5) KVQ_LAUNCH(6) KVQ_LAUNCH(7)
        KVQ_LAUNCH(8)
        default: return hipErrorInvalidValue;
    }
#undef KVQ_LAUNCH
    return hipGetLastError();
}

}  // namespace kvq
