// kvq_quantize.hip -- per-token norm, Lloyd-Max codes at the allocated widths and
// bit packing into 64-slot tiles (packed layout v1), for "RoPE-Aware Bit
// Allocation for KV-Cache Quantization" (abstract: TQ-MSE codes at the widths the
// Block-GTQ allocator assigns, kept in a packed cache).
//
// Two kernels write the same bytes.  The bulk kernel: one workgroup owns one
// (sequence, KV head, tile) -- the only writer of that tile during the call, so
// partially filled tiles are updated with plain read-modify-write -- with lane =
// token; norms, codes by binary search over the monotone threshold products, then
// the tile's K records, V runs and scales assembled dword by dword from the codes
// in LDS.  The append kernel (a few new tokens per sequence): one wave per (token,
// head), lane l holding coordinates 2l, 2l+1, the squared-norm tree by
// xor-butterflies (kvq_append.h).
#include "kvq_internal.h"
#include "kvq_append.h"

#pragma clang fp contract(off)

namespace kvq {

// Bulk quantize + pack, one workgroup per (sequence, KV head, tile), lane = token.
// The tile's fp16 rows are staged in LDS (rows 65 dwords apart: a coordinate read
// by 64 lanes touches distinct banks).  Norms: waves 0-3 sum the four 16-pair
// quarters of each K row, waves 4-7 those of V.  Codes: each wave takes a run of
// K-order fields (about an eighth of the work) and 16 of the V coordinates.  A
// field's width is the same for every lane, so the binary lifting runs without
// divergence, several fields of one width side by side, at a compile-time width.  Each coordinate is read by one wave
// only, which overwrites its fp16 value with the code; the store phase then builds
// every K record word and V run word in one thread from those code rows.
constexpr int kRowDw = kHeadDim / 2 + 1;
constexpr int kQWaves = 8;  // waves per workgroup
constexpr int kQThreads = 64 * kQWaves;
constexpr int kGroup = 4;   // K fields searched side by side
constexpr int kVGroup = 8;  // V coordinates searched side by side


// The top bit of a width-w code, as a byte offset into the width's threshold table: the
// middle threshold of every codebook is exactly +0 (the levels are symmetric), and
// s * (sig * 0) = +0 for the non-negative finite s and sig, so the first lifting step
// is the test x >= 0 (false for NaN, as the step is).
__device__ __forceinline__ uint32_t top_bit(float x, int w) { return x >= 0.f ? 4u << (w - 1) : 0u; }

// Binary lifting at a compile-time width W over G values side by side: c4 = 4 * (code so
// far); each step tries the next lower bit against the threshold product
// RN(s * RN(sig * t)), the threshold read at tw + c4 (tw: the width's LDS table, a
// constant that folds into the read's offset).  The top bit is the sign test.
template <int W, int G>
__device__ __forceinline__ void lift_codes(const float* tw, const float (&x)[G], const float (&sg)[G], float s,
                                           uint32_t (&c4)[G]) {
#pragma unroll
    for (int i = 0; i < G; ++i) c4[i] = top_bit(x[i], W);
#pragma unroll
    for (int sh = W - 2; sh >= 0; --sh) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const uint32_t cand = c4[i] | (4u << sh);
            const float a = *(const float*)((const char*)tw + cand);
            const float b = s * (sg[i] * a);
            if (x[i] >= b) c4[i] = cand;
        }
    }
}

// G key fields of width W for the lane's token; the codes overwrite the fields' fp16
// values in the lane's staged row.
template <int W, int G>
__device__ __forceinline__ void k_group(const uint32_t* fx, const float* fsig, uint16_t* krow, const float* thr,
                                        float sk) {
    uint32_t c[G], c4[G];
    float x[G], sg[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        c[i] = __builtin_amdgcn_readfirstlane(fx[i]) & 127u;
        sg[i] = fsig[i];
        x[i] = h2f(krow[c[i]]);
    }
    lift_codes<W, G>(thr + KVQ_CB_OFF(W), x, sg, sk, c4);
#pragma unroll
    for (int i = 0; i < G; ++i) krow[c[i]] = (uint16_t)(c4[i] >> 2);
}

template <int W>
__device__ __forceinline__ void k_group_w(int gn, const uint32_t* fx, const float* fsig, uint16_t* krow,
                                          const float* thr, float sk) {
    switch (gn) {
        case 1: k_group<W, 1>(fx, fsig, krow, thr, sk); break;
        case 2: k_group<W, 2>(fx, fsig, krow, thr, sk); break;
        case 3: k_group<W, 3>(fx, fsig, krow, thr, sk); break;
        default: k_group<W, kGroup>(fx, fsig, krow, thr, sk); break;
    }
}

// The wave's 16 value coordinates c0 .. c0 + 15 at the uniform width VB, eight side by
// side; slots outside the call get code 0.
template <int VB>
__device__ __forceinline__ void v_codes(uint16_t* vrow, const float* s_vsig, int c0, const float* thr, float sv,
                                        bool valid) {
#pragma unroll
    for (int g0 = 0; g0 < kHeadDim / kQWaves; g0 += kVGroup) {
        uint32_t c4[kVGroup];
        float x[kVGroup], sg[kVGroup];
#pragma unroll
        for (int i = 0; i < kVGroup; ++i) {
            x[i] = h2f(vrow[c0 + g0 + i]);
            sg[i] = s_vsig[c0 + g0 + i];
        }
        lift_codes<VB, kVGroup>(thr + KVQ_CB_OFF(VB), x, sg, sv, c4);
#pragma unroll
        for (int i = 0; i < kVGroup; ++i) vrow[c0 + g0 + i] = valid ? (uint16_t)(c4[i] >> 2) : (uint16_t)0;
    }
}

// Word k of coordinate c's run at width VB: bits [32k, 32k + 32) hold slots plo..phi,
// slot p's code at bit p*VB - 32k (the first one possibly cut at the word's start, the
// last at its end).  The slots' codes sit one staged row (2*kRowDw halves) apart, so
// every read after the first is at a constant offset from it.
template <int VB>
__device__ __forceinline__ uint32_t run_word(const uint32_t* s_v, int c, int k) {
    constexpr int kMaxSlots = 32 / VB + 2;  // slots a word can touch
    const int plo = 32 * k / VB, phi = min(kTile - 1, (32 * k + 31) / VB);
    const uint16_t* col = (const uint16_t*)s_v + c + plo * 2 * kRowDw;
    const int sh0 = plo * VB - 32 * k;  // in (-VB, 0]
    uint32_t val = (uint32_t)col[0] >> -sh0;
#pragma unroll
    for (int i = 1; i < kMaxSlots; ++i)
        if (plo + i <= phi) val |= (uint32_t)col[i * 2 * kRowDw] << (sh0 + i * VB);
    return val;
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
    __shared__ float s_thr[512];  // the codebook thresholds
    __shared__ float s_quarter[kQWaves][kTile];
    __shared__ float s_ks[kTile], s_vs[kTile];
    // K order, field f: coordinate | width << 7 | bit offset << 12, and the block's
    // sigma; padded so that a group read from any f stays in the arrays
    __shared__ uint32_t s_fx[kHeadDim + kGroup];
    __shared__ float s_fsig[kHeadDim + kGroup];
    __shared__ float s_vsig[kHeadDim];
    __shared__ int s_range[kQWaves + 1];  // wave w encodes fields [s_range[w], s_range[w+1])
    __shared__ uint8_t s_wfirst[65];      // the field holding bit 32k of the record (nf: none)
    __shared__ uint8_t s_cend[kHeadDim];  // field f -> the end of its width class in the K order

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
        int rank = 0, off = 0, ge = 0;  // ge: blocks at least as wide
        for (int wc = 16; wc >= 1; --wc) {
            const unsigned long long mk = __ballot(w == wc);
            if (wc > w) { rank += __popcll(mk); off += 2 * wc * __popcll(mk); }
            if (wc == w) { rank += __popcll(mk & below); off += 2 * wc * __popcll(mk & below); }
            if (wc >= w) ge += __popcll(mk);
        }
        const int nf = 2 * __popcll(__ballot(w > 0));
        s_wfirst[i] = (uint8_t)nf;
        if (i == 0) s_wfirst[64] = (uint8_t)nf;  // one past the longest record (64 words)
        if (w > 0) {
            const int pc = pairing == KVQ_PAIR_HALF ? i : 2 * i;
            const int qc = pairing == KVQ_PAIR_HALF ? i + kMaxBlocks : 2 * i + 1;
            s_cend[2 * rank] = s_cend[2 * rank + 1] = (uint8_t)(2 * ge);
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
            // both squares are exact in binary32, so the fused form rounds a^2 + b^2 once,
            // exactly as the separate products and sum do
            t[k] = __builtin_fmaf(a, a, b * b);
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
        // K: groups of up to kGroup consecutive fields of one width class (widths fall
        // along the K order), searched side by side, every field through all of its w
        // bits.  Width-16 fields keep the raw fp16 bits.
        const float sk = s_ks[lane];
        uint16_t* krow = (uint16_t*)(s_k + lane * kRowDw);
        const int f0 = __builtin_amdgcn_readfirstlane(s_range[wave]);
        const int f1 = __builtin_amdgcn_readfirstlane(s_range[wave + 1]);
        for (int f = f0; f < f1;) {
            const uint32_t fx0 = __builtin_amdgcn_readfirstlane(s_fx[f]);
            const int w = (fx0 >> 7) & 31;
            const int gn = min(min(kGroup, f1 - f), (int)__builtin_amdgcn_readfirstlane(s_cend[f]) - f);
            switch (w) {  // width 16 keeps the raw bits
                case 1: k_group_w<1>(gn, s_fx + f, s_fsig + f, krow, s_thr, sk); break;
                case 2: k_group_w<2>(gn, s_fx + f, s_fsig + f, krow, s_thr, sk); break;
                case 3: k_group_w<3>(gn, s_fx + f, s_fsig + f, krow, s_thr, sk); break;
                case 4: k_group_w<4>(gn, s_fx + f, s_fsig + f, krow, s_thr, sk); break;
                case 5: k_group_w<5>(gn, s_fx + f, s_fsig + f, krow, s_thr, sk); break;
                case 6: k_group_w<6>(gn, s_fx + f, s_fsig + f, krow, s_thr, sk); break;
                case 7: k_group_w<7>(gn, s_fx + f, s_fsig + f, krow, s_thr, sk); break;
                case 8: k_group_w<8>(gn, s_fx + f, s_fsig + f, krow, s_thr, sk); break;
                default: break;
            }
            f += gn;
        }

        // V: kVGroup coordinates at a time; slots outside the call get code 0 (16-bit
        // V keeps the raw rows, whose invalid slots the run builder skips)
        const float sv = s_vs[lane];
        uint16_t* vrow = (uint16_t*)(s_v + lane * kRowDw);
        const int c0 = (kHeadDim / kQWaves) * wave;
        switch (v_bits) {  // 16-bit values keep the raw rows (the run builder skips invalid slots)
            case 1: v_codes<1>(vrow, s_vsig, c0, s_thr, sv, valid); break;
            case 2: v_codes<2>(vrow, s_vsig, c0, s_thr, sv, valid); break;
            case 3: v_codes<3>(vrow, s_vsig, c0, s_thr, sv, valid); break;
            case 4: v_codes<4>(vrow, s_vsig, c0, s_thr, sv, valid); break;
            case 5: v_codes<5>(vrow, s_vsig, c0, s_thr, sv, valid); break;
            case 6: v_codes<6>(vrow, s_vsig, c0, s_thr, sv, valid); break;
            case 7: v_codes<7>(vrow, s_vsig, c0, s_thr, sv, valid); break;
            case 8: v_codes<8>(vrow, s_vsig, c0, s_thr, sv, valid); break;
            default: break;
        }
    }
    __syncthreads();

    // ---- phase 3: the tile's records (valid slots), runs and scales
    // K record word k of slot `lane`: the field holding bit 32k (s_wfirst[k]) and every
    // later one that starts before bit 32k + 32 -- up to the field holding bit 32k + 32
    // when it starts inside the word -- each field's code shifted to its offset
    uint32_t* krec = (uint32_t*)tile;
    {
        const uint16_t* krow = (const uint16_t*)(s_k + lane * kRowDw);
        const int nf = __builtin_amdgcn_readfirstlane(s_range[kQWaves]);
        // waves 4-7 take the first words: waves 0-3 take the second round of run words below
        for (int k = (wave + kQWaves / 2) % kQWaves; k < RW; k += kQWaves) {
            const int lo = 32 * k;
            uint32_t val = 0u;
            const int fa = __builtin_amdgcn_readfirstlane(s_wfirst[k]);
            int fb = __builtin_amdgcn_readfirstlane(s_wfirst[k + 1]);
            if (fb < nf && (int)((__builtin_amdgcn_readfirstlane(s_fx[fb]) >> 12) & 2047) < lo + 32) ++fb;
            if (fa < nf) {
                const uint32_t fx0 = __builtin_amdgcn_readfirstlane(s_fx[fa]);
                val = (uint32_t)krow[fx0 & 127] >> (lo - (int)((fx0 >> 12) & 2047));
                int f = fa + 1;
                for (; f + kGroup <= fb; f += kGroup) {
                    uint32_t fx[kGroup], code[kGroup];
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) fx[i] = __builtin_amdgcn_readfirstlane(s_fx[f + i]);
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) code[i] = krow[fx[i] & 127];
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) val |= code[i] << ((int)((fx[i] >> 12) & 2047) - lo);
                }
                for (; f < fb; ++f) {
                    const uint32_t fx1 = __builtin_amdgcn_readfirstlane(s_fx[f]);
                    val |= (uint32_t)krow[fx1 & 127] << ((int)((fx1 >> 12) & 2047) - lo);
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
            switch (v_bits) {
                case 1: val = run_word<1>(s_v, c, k); break;
                case 2: val = run_word<2>(s_v, c, k); break;
                case 3: val = run_word<3>(s_v, c, k); break;
                case 4: val = run_word<4>(s_v, c, k); break;
                case 5: val = run_word<5>(s_v, c, k); break;
                case 6: val = run_word<6>(s_v, c, k); break;
                case 7: val = run_word<7>(s_v, c, k); break;
                default: val = run_word<8>(s_v, c, k); break;
            }
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
    append_token(kx, vx, stride_tok, stride_head, first_slot, n_new, src_row0, max_new, capacity, k_bits, k_sigma,
                 v_sigma, cache, seq_byte_off, pairing, k_budget, v_bits, step_len, app, blockIdx.z, blockIdx.y,
                 blockIdx.x, threadIdx.x);
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

}  // namespace kvq
