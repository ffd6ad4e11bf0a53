// kvq_decode_mfma.h -- packed-cache GQA decode attention on the CDNA4 matrix
// cores (gfx950), for the packed-cache serving path of "RoPE-Aware Bit
// Allocation for KV-Cache Quantization" (abstract).
//
// Per 64-slot tile, one wave computes
//   z_t = s_t * sum_c (q_c sigma_c scale log2e) level[code_{t,c}]               (QK)
//   o  += sum_t 2^(z_t - m) s^V_t level[vcode_{t,c}]   (times sigma^V_c at the end)  (PV)
// with the levels (exact binary16) as matrix operands and the fp32 factors
// q.sigma and p.s^V split into binary16 hi + lo parts, so products keep ~22 bits.
//
// QK uses v_mfma_f32_32x32x16_f16 with a block-diagonal B operand: lane l decodes
// one token (slot qslot(l)), and all 64 lanes decode the SAME 8 K-order
// coordinates per instruction (K widths are per (layer, head), so field offsets
// and widths are wave-uniform).  Lanes 0-31 feed token set 0 into k-slots 0-7 and
// lanes 32-63 feed token set 1 into k-slots 8-15; B columns 0-15 read only k-slots
// 0-7 and columns 16-31 only k-slots 8-15, each column being (hi|lo, head).  Since
// the K order sorts blocks by width, the coordinates are taken one width class at
// a time, 8 fields per instruction with compile-time offsets (the last unit of a
// class is padded with zero q in the operand, never in the cache).
//
// The 32x32 accumulator then holds, in lane l, 16 logits of column l%32 for slots
// 16*(l/16) + i, i = 0..15 -- exactly the A-operand layout of the PV product
// v_mfma_f32_16x16x32_f16 (row = l%16 = (hi|lo, head), k = 8*(l/16) + j), so the
// softmax weights never leave registers.  The PV B operand of lane l is 16
// consecutive slots of one coordinate, one contiguous 16*v-bit piece of a V run.
// Codes become binary16 levels through LDS tables: two codes per lookup (a dword
// of two levels) for widths <= 5, one code per lookup for widths 6..8.
//
// The running max is a lazy reference: it only moves (and the accumulators are
// only rescaled) when a head's tile max exceeds it by more than 8 (log2 units),
// so p <= 2^8.  The binary16 PV operand p.s^V must stay finite for any value norm
// s^V a binary16 row can have (up to 65504 sqrt(128)), so the reference also carries
// a wave-uniform power of two: weights are taken against R = m + e with the integer
// e >= 0 the least that keeps every s^V seen so far at most 2^(7+e); p.s^V.2^-e then
// stays below 2^15, and o and l, both relative to R, are rescaled exactly as when m
// moves.  With value norms below 2^7 e stays 0.  Each wave loads tile n+1 while it
// computes tile n.
//
// 16-bit values (the K-only mode, V = 16) are their own PV operands: each lane loads
// its 16 slots of a coordinate's run straight from the cache into registers (three
// batches per tile, the first in flight during QK), with value norm and block scale
// taken as 1; only the tile's token scales pass through LDS.
#pragma once
#include <math.h>

#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxUnits = 24;  // 128 coordinates in 8-wide units, plus one partial unit per width class
constexpr int kWaves = 4;
constexpr float kRescaleSlack = 8.f;
constexpr int kVNormExp = 7;  // value norms are kept at most 2^kVNormExp after the power-of-two shift

// level tables: pairs (widths 1..5): entry a | b << w -> half2(level_w[a], level_w[b]);
// singles (widths 6..8)
constexpr int kPairMax = 5;
__host__ __device__ constexpr int pair_off(int w) { return w == 1 ? 0 : w == 2 ? 4 : w == 3 ? 20 : w == 4 ? 84 : 340; }
constexpr int kPairEntries = 1364;
__host__ __device__ constexpr int single_off(int w) { return w == 6 ? 0 : w == 7 ? 64 : 192; }
constexpr int kSingleEntries = 448;

struct alignas(16) LevelTables {
    uint32_t pair[kPairEntries];
    uint16_t single[kSingleEntries];
};
static_assert(sizeof(LevelTables) % 16 == 0, "tables are copied to LDS in 16-byte pieces");

constexpr uint16_t kLevelsInit[510] = {KVQ_LEVELS_FP16_LIST};
constexpr LevelTables make_level_tables() {
    LevelTables t{};
    for (int w = 1; w <= kPairMax; ++w)
        for (int e = 0; e < (1 << (2 * w)); ++e) {
            const int a = e & ((1 << w) - 1), b = e >> w;
            t.pair[pair_off(w) + e] =
                (uint32_t)kLevelsInit[KVQ_CB_OFF(w) + a] | ((uint32_t)kLevelsInit[KVQ_CB_OFF(w) + b] << 16);
        }
    for (int w = kPairMax + 1; w <= 8; ++w)
        for (int e = 0; e < (1 << w); ++e) t.single[single_off(w) + e] = kLevelsInit[KVQ_CB_OFF(w) + e];
    return t;
}
static __device__ const LevelTables g_level_tables = make_level_tables();

union H8 {
    half8 h;
    uint32_t u[4];
    uint16_t s[8];
};

__device__ __forceinline__ uint32_t alignbit(uint32_t hi, uint32_t lo, uint32_t s) {
    return __builtin_amdgcn_alignbit(hi, lo, s);
}

struct MfmaSmem {
    LevelTables tab;
    // binary16 hi/lo of q.sigma.scale by padded position: width class w occupies whole
    // 8-position units (its last unit zero-padded), classes in descending width
    alignas(16) uint16_t qsplit[2][8][8 * kMaxUnits + 8];  // rows 400 B apart: the 16 rows read by one
                                                          // b128 load fall in distinct LDS banks
    alignas(16) uint16_t qzero[8 * kMaxUnits + 8];         // a zero row as long: the off-diagonal B rows
    alignas(16) float alpha[kWaves][8];
    alignas(16) float wm[8][kWaves];  // per head: each wave's reference R (log2 units)
    alignas(16) float wl[8][kWaves];  // ... and its sum of weights
    uint32_t arec[16];                // the appended token's K record, assembled
};
// the waves' unnormalised outputs [wave][coordinate][head], combined at the end in
// the (then idle) tile buffers: the shared buffers hold at least this much
typedef float WaveOut[kWaves][kHeadDim][8];


// byte offset 4 * (bits [r, r + n) of x), for a table of dwords
template <int R, int N>
__device__ __forceinline__ uint32_t field_x4(uint32_t x) {
    constexpr uint32_t m = ((1u << N) - 1u) << 2;
    if (R >= 2) return (x >> (R - 2)) & m;
    return (x << (2 - R)) & m;
}
// byte offset 2 * (bits [r, r + n) of x), for a table of halves
template <int R, int N>
__device__ __forceinline__ uint32_t field_x2(uint32_t x) {
    constexpr uint32_t m = ((1u << N) - 1u) << 1;
    if (R >= 1) return (x >> (R - 1)) & m;
    return (x << 1) & m;
}
__device__ __forceinline__ uint32_t lds_u32(const void* base, uint32_t byte_off) {
    return *(const uint32_t*)((const char*)base + byte_off);
}
__device__ __forceinline__ uint32_t lds_u16(const void* base, uint32_t byte_off) {
    return *(const uint16_t*)((const char*)base + byte_off);
}

// Two equal-width fields at bit offset REL of the 64-bit window hi:lo, returned
// as two binary16 levels in one dword.
template <int W, int REL>
__device__ __forceinline__ uint32_t decode_pair(const LevelTables& t, uint32_t lo, uint32_t hi) {
    if (W <= kPairMax) {
        const uint32_t* base = t.pair + pair_off(W);
        if (REL >= 32) return lds_u32(base, field_x4<(REL >= 32 ? REL - 32 : 0), 2 * W>(hi));
        if (REL + 2 * W <= 32) return lds_u32(base, field_x4<(REL < 32 ? REL : 0), 2 * W>(lo));
        return lds_u32(base, field_x4<0, 2 * W>(alignbit(hi, lo, REL)));
    } else {
        const uint16_t* base = t.single + single_off(W);
        uint32_t xa, xb;
        if (REL >= 32) { xa = hi >> (REL - 32); }
        else if (REL + W <= 32) { xa = lo >> REL; }
        else { xa = alignbit(hi, lo, REL); }
        if (REL + W >= 32) { xb = hi >> (REL + W - 32); }
        else if (REL + 2 * W <= 32) { xb = lo >> (REL + W); }
        else { xb = alignbit(hi, lo, REL + W); }
        return lds_u16(base, field_x2<0, W>(xa)) | (lds_u16(base, field_x2<0, W>(xb)) << 16);
    }
}

// Both operands of unit j of a width class: the window of 8 fields -> A, the q split
// of the lane's B column -> B (the column's zero row off the diagonal)
template <int W, int RD>
__device__ __forceinline__ void qk_unit(const MfmaSmem& sm, const uint32_t (&rec)[RD + 2], int st,
                                        const uint16_t* qrow, H8& a, H8& b) {
    const int d = min(st >> 5, RD > 0 ? RD - 1 : 0);
    const uint32_t sh = (uint32_t)(st & 31);
    const uint32_t d0 = rec[d], d1 = rec[d + 1];
    const uint32_t lo = alignbit(d1, d0, sh);
    const uint32_t hi = W <= 4 ? 0u : alignbit(rec[d + 2], d1, sh);
    a.u[0] = decode_pair<W, 0>(sm.tab, lo, hi);
    a.u[1] = decode_pair<W, 2 * W>(sm.tab, lo, hi);
    a.u[2] = decode_pair<W, 4 * W>(sm.tab, lo, hi);
    a.u[3] = decode_pair<W, 6 * W>(sm.tab, lo, hi);
    const uint4 q4 = *(const uint4*)qrow;
    b.u[0] = q4.x; b.u[1] = q4.y; b.u[2] = q4.z; b.u[3] = q4.w;
}

// QK over the units of one width class, two units per step into two accumulators
// (independent MFMA chains, both units' lookups in flight together).  qb: the lane's
// q split row (the zero row off the diagonal); unit u's 8 positions sit 16 bytes after
// unit u - 1's.
template <int W, int RD>
__device__ __forceinline__ void qk_class(const MfmaSmem& sm, const uint32_t (&rec)[RD + 2], int start, int units,
                                         int ubase, const uint16_t* qb, floatx16& acc0, floatx16& acc1) {
    const char* qc = (const char*)qb;
    int j = 0;
    for (; j + 1 < units; j += 2) {
        H8 a0, b0, a1, b1;
        qk_unit<W, RD>(sm, rec, start + j * 8 * W, (const uint16_t*)(qc + 16u * (ubase + j)), a0, b0);
        qk_unit<W, RD>(sm, rec, start + (j + 1) * 8 * W, (const uint16_t*)(qc + 16u * (ubase + j + 1)), a1, b1);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0.h, b0.h, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1.h, b1.h, acc1, 0, 0, 0);
    }
    if (j < units) {
        H8 a0, b0;
        qk_unit<W, RD>(sm, rec, start + j * 8 * W, (const uint16_t*)(qc + 16u * (ubase + j)), a0, b0);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0.h, b0.h, acc0, 0, 0, 0);
    }
}

// PV B operand (16 consecutive slots of one coordinate) from the lane's raw words
template <int V>
__device__ __forceinline__ void decode_v(const LevelTables& t, const uint32_t* raw, uint32_t sh, H8& b0, H8& b1) {
    constexpr int NW = (16 * V + 31) / 32;
    uint32_t nw[NW + 1];
#pragma unroll
    for (int k = 0; k < NW; ++k) nw[k] = alignbit(raw[k + 1], raw[k], sh);
    nw[NW] = 0;
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
        const int bit = 2 * V * pr;
        const int k = bit >> 5, r = bit & 31;
        uint32_t val;
        if (V <= kPairMax) {
            const uint32_t* base = t.pair + pair_off(V);
            const uint32_t src = (r + 2 * V <= 32) ? (nw[k] >> r) : alignbit(nw[k + 1], nw[k], r);
            val = lds_u32(base, (src << 2) & (((1u << (2 * V)) - 1u) << 2));
        } else {
            const uint16_t* base = t.single + single_off(V);
            const int bit2 = bit + V, k2 = bit2 >> 5, r2 = bit2 & 31;
            const uint32_t sa = (r + V <= 32) ? (nw[k] >> r) : alignbit(nw[k + 1], nw[k], r);
            const uint32_t sb = (r2 + V <= 32) ? (nw[k2] >> r2) : alignbit(nw[k2 + 1], nw[k2], r2);
            val = lds_u16(base, (sa << 1) & (((1u << V) - 1u) << 1)) |
                  (lds_u16(base, (sb << 1) & (((1u << V) - 1u) << 1)) << 16);
        }
        if (pr < 4) b0.u[pr] = val; else b1.u[pr - 4] = val;
    }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14)
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)
constexpr int wait_vm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) & 3) << 14; }  // vmcnt(n)

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4; M0 holds the wave-uniform LDS base).  Written as asm so
// that the compiler does not order every later LDS read behind it: the caller
// waits for it explicitly (vmcnt) before reading the buffer, and issues it only
// after its own reads of that buffer have returned (lgkmcnt).  The decode kernel
// reads each tile once and marks its loads non-temporal (STREAM), so the packed
// stream does not push a launch's small shared inputs (level tables, queries,
// scales) out of L2 between launches; the prefill kernel re-reads tiles from many
// workgroups and keeps them cacheable.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is reserved, and this asm does overwrite it
template <bool STREAM = false>
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
    if (STREAM)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                     :
                     : "v"(gptr), "s"(lds_base)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :
                     : "v"(gptr), "s"(lds_base)
                     : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier that orders LDS only: its fences wait for this wave's LDS
// operations (lgkmcnt) and not for its outstanding global loads, so a tile's DMA in
// flight does not hold the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int V, int RD, bool ROT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void decode_mfma_kernel(
    const uint16_t* __restrict__ q, uint8_t* __restrict__ cache, const int64_t* __restrict__ seq_byte_off,
    const int32_t* __restrict__ seq_len, int64_t max_len, int64_t capacity, const uint8_t* __restrict__ k_bits,
    const float* __restrict__ k_sigma, const float* __restrict__ v_sigma, float scale_log2, int n_q, int g,
    int pairing, int k_budget, int tiles_per_split, int n_split, float* __restrict__ ws, AppendArgs app) {
    // 16-bit values (the K-only mode) need no decoding: the lanes load their PV operands
    // straight into registers, and only the tile's scales are staged in LDS
    constexpr bool V16 = V == 16;
    constexpr int SK = 4 * RD;                   // K record bytes
    constexpr int KB = kTile * SK;               // K section of a tile
    constexpr int VR = kHeadDim * 8 * V;         // V runs of a tile
    constexpr int VB = VR + 2 * kTile * 4;       // V runs and scales
    constexpr int VL = V16 ? 2 * kTile * 4 : VB;  // the part of them staged in LDS
    constexpr int TB = KB + VB;
    constexpr int KI = RD / 4;                   // 16-byte DMA instructions of a K section
    constexpr int VI = (VL / 16 + 63) / 64;      // ... of a V section
    constexpr int WB = 2 * KB + VL;              // per wave: two K buffers, one V buffer
    constexpr int NW = (16 * V + 31) / 32;       // words of one lane's V piece
    constexpr int BUF = kWaves * WB > (int)sizeof(WaveOut) ? kWaves * WB : (int)sizeof(WaveOut);
    __shared__ MfmaSmem sm;
    __shared__ __attribute__((aligned(16))) uint8_t bufs[BUF];
    // grid (KV head, chunk, sequence): dispatch walks the heads fastest, so a
    // sequence's last chunks -- the short tail chunk in particular -- go out last and
    // land beside full workgroups instead of displacing one
    const int kvh = blockIdx.x, split = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (app.window > 0 && split >= n_split - window_chunks(app.window)) {  // the fp16 window's chunks
        window_chunk<8>(app, q, n_q, g, s, kvh, seq_len, scale_log2, ws, n_split,
                        split - (n_split - window_chunks(app.window)), (float*)bufs);
        return;
    }

    // ---- every global load of the prologue goes out before anything waits on one
    // (no load sits under a branch, so none is waited for on its own)
    const int64_t len_raw = seq_len[s];
    const int64_t seq_off = seq_byte_off[s];
    const int my_w = k_bits[kvh * kMaxBlocks + lane];
    const float my_ksig = k_sigma[kvh * kMaxBlocks + lane];
    const int vs_blk = pairing == KVQ_PAIR_HALF ? (tid & (kMaxBlocks - 1)) : ((tid >> 1) & (kMaxBlocks - 1));
    // the value block scale of coordinate tid % 128: the combine's thread (half, c) scales
    // coordinate c by it (both halves map c to the same block)
    const float my_vsig = v_sigma[kvh * kMaxBlocks + vs_blk];
    const int qp = pairing == KVQ_PAIR_HALF ? lane : 2 * lane;
    const int qq = pairing == KVQ_PAIR_HALF ? lane + kMaxBlocks : 2 * lane + 1;
    uint32_t qv[2][2];  // heads wave and wave + 4 (clamped; unused past the group): coordinates qp, qq
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int hh = min(wave + kWaves * e, g - 1);
        const uint16_t* qrow = q + ((int64_t)s * n_q + kvh * g + hh) * kHeadDim;
        qv[e][0] = qrow[qp];
        qv[e][1] = qrow[qq];
    }
    // the rotated variant's step: the key signs of the lane's two coordinates (the
    // queries and the new key are rotated here), and the value signs when values rotate
    uint32_t ksg_p = 0, ksg_q = 0, vsg_p = 0, vsg_q = 0;
    if constexpr (ROT) {
        ksg_p = app.k_signs[kvh * kHeadDim + qp];
        ksg_q = app.k_signs[kvh * kHeadDim + qq];
        const uint8_t* vsg = app.v_signs != nullptr ? app.v_signs : app.k_signs;
        vsg_p = vsg[kvh * kHeadDim + qp];
        vsg_q = vsg[kvh * kHeadDim + qq];
    }
    constexpr int kTabChunks = (int)(sizeof(LevelTables) / 16);
    static_assert(kTabChunks > 256 && kTabChunks <= 512, "the level tables are staged in two 16-byte pieces per thread");
    const uint4* tsrc = (const uint4*)&g_level_tables;
    const uint4 tab0 = tsrc[tid];
    const uint4 tab1 = tsrc[min(tid + 256, kTabChunks - 1)];

    // the step's new token (coordinates 2l, 2l+1 for its norm; block l's p, q for its codes)
    uint32_t nk_pair = 0, nv_pair = 0, nk_p = 0, nk_q = 0, nv_p = 0, nv_q = 0;
    float my_vsig_blk = 0.f;
    if (app.k != nullptr) {
        // with a window the token is the ring row leaving it (needs the length first)
        const int64_t ring_row = app.window > 0 && len_raw > 0 ? ((len_raw - 1) % app.window) * kHeadDim : 0;
        const uint16_t* kr = app.k + (int64_t)s * app.stride_seq + (int64_t)kvh * app.stride_head + ring_row;
        const uint16_t* vr = app.v + (int64_t)s * app.stride_seq + (int64_t)kvh * app.stride_head + ring_row;
        nk_pair = *(const uint32_t*)(kr + 2 * lane);
        nv_pair = *(const uint32_t*)(vr + 2 * lane);
        nk_p = kr[qp]; nk_q = kr[qq];
        nv_p = vr[qp]; nv_q = vr[qq];
        my_vsig_blk = v_sigma[kvh * kMaxBlocks + lane];
    }

    const int64_t len = min(max(len_raw - app.window, (int64_t)0), max_len);  // packed tokens
    const int64_t n_tiles_seq = (len + kTile - 1) / kTile;
    const int64_t t0 = (int64_t)split * tiles_per_split;
    const int64_t t1 = min(t0 + tiles_per_split, n_tiles_seq);
    // the wave whose tiles include slot len-1 appends the new token there first
    const int64_t tail_tau = (len - 1) / kTile;
    const bool wg_appends = app.k != nullptr && len > 0 && tail_tau >= t0 && tail_tau < t1;
    const int app_wave = (int)((tail_tau - t0) % kWaves);
    const bool appender = wg_appends && app_wave == wave;
    float thr_a = 0.f, thr_b = 0.f;  // the codebook thresholds, staged for the appender by the whole group
    if (wg_appends) {
        thr_a = c_thresholds[tid];
        thr_b = c_thresholds[min(tid + 256, 509)];
    }

    // lane roles
    const int col = lane & 31;
    const bool bdiag = (col >> 4) == (lane >> 5);
    const int m = lane & 31;
    const int qslot = 16 * (2 * ((m >> 2) & 1) + (lane >> 5)) + 4 * (m >> 3) + (m & 3);  // QK token
    const int grp = lane >> 4;       // PV k group: slots 16*grp .. 16*grp+15
    const int row = lane & 15;       // PV row = (hi|lo) * 8 + head
    const float mlo = row >= 8 ? -1.f : 0.f;  // lo rows subtract the hi part of each weight

    const uint8_t* head_base = cache + seq_off + (int64_t)kvh * (capacity / kTile) * TB;
    uint8_t* wbuf = bufs + wave * WB;
    const uint32_t wbuf_lds = (uint32_t)(uintptr_t)(lds_u8*)wbuf;

    // Tile DMA.  A K section goes to K buffer kb with record chunks chunk-major
    // (chunk k of record r at 16*(64*k + r)); a V section (runs, then scales) goes
    // linearly to the V buffer.  Each wave issues, in order: K(n+1) once tile n's V
    // section has landed and V(n+1) once tile n's V reads have returned (the first
    // tile: K in the prologue, V once that K is in), so at the start of a tile its K
    // section is complete once at most VI loads are outstanding, and its V section
    // once none are.
    auto dma_k = [&](int64_t tau, int kb) {
        const uint8_t* tile = head_base + tau * TB;
#pragma unroll
        for (int k = 0; k < KI; ++k) dma16<true>(tile + lane * SK + 16 * k, wbuf_lds + kb * KB + 1024 * k);
    };
    auto dma_v = [&](int64_t tau) {
        const uint8_t* vsec = head_base + tau * TB + KB + (V16 ? VR : 0);
#pragma unroll
        for (int j = 0; j < VI; ++j) {
            const int ch = 64 * j + lane;
            if (64 * j + 63 < VL / 16 || ch < VL / 16) dma16<true>(vsec + 16 * ch, wbuf_lds + 2 * KB + 1024 * j);
        }
    };
    // 16-bit values: the lane's PV operands for coordinates 16*ct + row, ct in
    // [C0, C1), slots 16*grp .. 16*grp + 15 (32 bytes of each coordinate's run),
    // straight into registers.  They go out in three batches -- before QK, once QK is
    // done, once the weights are -- so that no more are held than the phase allows.
    constexpr int kPre = 3, kMid = 3;  // coordinate tiles of the first two batches
    auto load_v16 = [&](int64_t tau, auto c0, auto c1, u32x4 (&vr)[16]) {
        constexpr int C0 = decltype(c0)::value, C1 = decltype(c1)::value;
        const u32x4* vg = (const u32x4*)(head_base + tau * TB + KB + row * (8 * V) + 2 * V * grp);
#pragma unroll
        for (int ct = C0; ct < C1; ++ct) {
            vr[2 * ct] = __builtin_nontemporal_load(vg + ct * 16 * (8 * V) / 16);
            vr[2 * ct + 1] = __builtin_nontemporal_load(vg + ct * 16 * (8 * V) / 16 + 1);
        }
    };
    using IC0 = std::integral_constant<int, 0>;
    using IC1 = std::integral_constant<int, kPre>;
    using IC2 = std::integral_constant<int, kPre + kMid>;
    using IC3 = std::integral_constant<int, 8>;
    constexpr bool kStageInK1 = KB >= 510 * 4;  // see the staging area below
    int64_t tau = t0 + wave;

    // ------------------------------------------------------------------ prologue
    // the appender's staging area for the thresholds: its second K buffer when that
    // holds them (idle until its first tile starts), else its own buffers (which then
    // fill only after the append) or the spare end of the shared buffer
    static_assert(WB >= 510 * 4 || BUF - kWaves * WB >= 510 * 4, "no room to stage the thresholds");
    static_assert(BUF >= (8 * kHeadDim + 2 * 8 * kWindowChunk) * 4, "the window chunk's scratch lives in the tile buffers");
    float* const s_thr = (float*)(kStageInK1 ? bufs + app_wave * WB + KB
                                            : WB >= 510 * 4 ? bufs + app_wave * WB : bufs + kWaves * WB);
    if (wg_appends) {
        s_thr[tid] = thr_a;
        if (tid + 256 < 510) s_thr[tid + 256] = thr_b;
    }
    ((uint4*)&sm.tab)[tid] = tab0;
    if (tid + 256 < kTabChunks) ((uint4*)&sm.tab)[tid + 256] = tab1;
    {
        uint4* qz = (uint4*)&sm.qsplit[0][0][0];
        for (int i = tid; i < (int)(sizeof(sm.qsplit) / 16); i += 256) qz[i] = uint4{0, 0, 0, 0};
        if (tid < (int)(sizeof(sm.qzero) / 16)) ((uint4*)sm.qzero)[tid] = uint4{0, 0, 0, 0};
    }
    // width classes (descending): every wave ranks the blocks; a block's two fields sit
    // at its rank within its class.  Wave w fills the q split of heads w, w+4.
    int my_pos = 0, my_koff = 0;  // q split position and K record bit offset of block `lane`
    int cstart[9], cunits[9], cubase[9];
    {
        const unsigned long long below = (1ull << lane) - 1ull;
        int start = 0, ubase = 0;
#pragma unroll
        for (int w = 8; w >= 1; --w) {
            const unsigned long long mk = __ballot(my_w == w);
            const int nfw = 2 * __popcll(mk), units = (nfw + 7) >> 3;
            cstart[w] = start;
            cunits[w] = units;
            cubase[w] = ubase;
            if (my_w == w) {
                my_pos = 8 * ubase + 2 * __popcll(mk & below);
                my_koff = start + 2 * w * __popcll(mk & below);
            }
            start += nfw * w;
            ubase += units;
        }
    }
    if constexpr (ROT) {
        // q_rot = RN16(RN32(RN32(S) * sigma_rot)), S = H (sg * q) exact: the lane's two
        // coordinates of heads wave and wave + 4
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float a, b;
            rotated_pair_f32(qv[e][0], qv[e][1], ksg_p, ksg_q, lane, a, b);
            qv[e][0] = __builtin_bit_cast(uint16_t, (_Float16)(a * kRotSigma));
            qv[e][1] = __builtin_bit_cast(uint16_t, (_Float16)(b * kRotSigma));
        }
    }
    lds_barrier();  // zeroed q split before it is filled
    if (my_w > 0) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int hh = wave + kWaves * e;
            if (hh >= g) continue;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const float v = h2f(qv[e][f]) * my_ksig * scale_log2;
                const _Float16 hi = (_Float16)v;
                const _Float16 lo = (_Float16)(v - (float)hi);
                sm.qsplit[0][hh][my_pos + f] = __builtin_bit_cast(uint16_t, hi);
                sm.qsplit[1][hh][my_pos + f] = __builtin_bit_cast(uint16_t, lo);
            }
        }
    }
    // The first tile's DMA goes out once the prologue's own loads have been consumed:
    // loads complete in issue order, so a wait for any load issued before the DMA
    // but used after it would also wait for the whole tile.  The barriers here order
    // LDS only, so each wave starts on its tile as soon as its own K section lands.
    if (tau < t1 && (kStageInK1 || !appender)) dma_k(tau, 0);
    lds_barrier();
    // B operand rows: the lane's column (hi|lo, head) on the diagonal, else the zero row
    // (as long as a q split row, so every lane's unit address is one add)
    const uint16_t* qb = bdiag ? &sm.qsplit[(col >> 3) & 1][col & 7][0] : &sm.qzero[0];

    // ---- the step's append (one wave): quantize and pack the new token for slot
    // len-1 exactly as the quantize path does.  The bytes go into the LDS copy of
    // the tail tile when it arrives, and to the cache after the tiles.
    const int tail_p = (int)((len - 1) & (kTile - 1));
    uint32_t ap_rec = 0, ap_vcp = 0, ap_vcq = 0;
    float ap_sk = 0.f, ap_sv = 0.f;
    if (appender) {
        uint32_t* s_rec = sm.arec + 0;
        if (lane < 16) s_rec[lane] = 0;
        ap_sk = token_norm(nk_pair);
        ap_sv = token_norm(nv_pair);
        uint32_t kcp, kcq;
        if constexpr (ROT) {
            // rotated coordinates at the uniform width, sigma 1 (the 1/sqrt(128) is in
            // the comparison), the unrotated row's norm
            float a, b;
            rotated_pair_f32(nk_p, nk_q, ksg_p, ksg_q, lane, a, b);
            kcp = code_of(s_thr, a, my_w, 1.f, ap_sk);
            kcq = code_of(s_thr, b, my_w, 1.f, ap_sk);
            if (app.v_signs != nullptr) {
                float c, d;
                rotated_pair_f32(nv_p, nv_q, vsg_p, vsg_q, lane, c, d);
                ap_vcp = code_of(s_thr, c, V, 1.f, ap_sv);
                ap_vcq = code_of(s_thr, d, V, 1.f, ap_sv);
            } else {
                ap_vcp = encode(s_thr, nv_p, V, my_vsig_blk, ap_sv);
                ap_vcq = encode(s_thr, nv_q, V, my_vsig_blk, ap_sv);
            }
        } else {
            kcp = encode(s_thr, nk_p, my_w, my_ksig, ap_sk);
            kcq = encode(s_thr, nk_q, my_w, my_ksig, ap_sk);
            ap_vcp = encode(s_thr, nv_p, V, my_vsig_blk, ap_sv);
            ap_vcq = encode(s_thr, nv_q, V, my_vsig_blk, ap_sv);
        }
        if constexpr (V16) {
            // 16-bit values go into the cache now: the tail tile's operands are loaded
            // from there, after the first tile's wait for every load (vmcnt counts
            // these atomics too) -- the tail tile is this wave's alone
            uint32_t* vrun = (uint32_t*)((uint8_t*)head_base + tail_tau * TB + KB);
            const int vk = tail_p >> 1, vsh = 16 * (tail_p & 1);
            if (ap_vcp != 0) atomicOr(vrun + qp * 2 * V + vk, ap_vcp << vsh);
            if (ap_vcq != 0) atomicOr(vrun + qq * 2 * V + vk, ap_vcq << vsh);
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        if (my_w > 0) {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const uint32_t code = f ? kcq : kcp;
                const int off = my_koff + f * my_w, k = off >> 5, sh = off & 31;
                atomicOr(&s_rec[k], code << sh);
                if (sh + my_w > 32) atomicOr(&s_rec[k + 1], code >> (32 - sh));
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        ap_rec = lane < RD ? s_rec[lane] : 0u;
        // the staging reads have returned: the buffers may refill
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        if (!kStageInK1 && tau < t1) dma_k(tau, 0);
        if (app.window > 0 && app.k_new != nullptr) {  // the step's new token takes the ring row just read
            const int64_t nr = (int64_t)s * app.new_stride_seq + (int64_t)kvh * app.new_stride_head + 2 * lane;
            const uint32_t kn = *(const uint32_t*)(app.k_new + nr);
            const uint32_t vn = *(const uint32_t*)(app.v_new + nr);
            const int64_t rr = (int64_t)s * app.stride_seq + (int64_t)kvh * app.stride_head +
                               ((len_raw - 1) % app.window) * kHeadDim + 2 * lane;
            *(uint32_t*)(app.ring_k + rr) = kn;
            *(uint32_t*)(app.ring_v + rr) = vn;
        }
    }

    floatx4 o[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) o[ct] = floatx4{0.f, 0.f, 0.f, 0.f};
    float mref = -INFINITY, lrun = 0.f;
    float vexp = 0.f, vlim = (float)(1 << kVNormExp);  // the reference's power of two e, and 2^(7+e)

    // ------------------------------------------------------------------ tiles
    int kb = 0;
    bool first = true;
    for (; tau < t1; tau += kWaves) {
        const int nvalid = (int)min((int64_t)kTile, len - tau * kTile);
        const bool more = tau + kWaves < t1;
        // K section landed: the lane's record to registers, then the next K section
        // into the other K buffer.  The first tile's V section is requested only once
        // its K section is in (the start of the launch asks for K sections alone, so
        // they arrive sooner); later V sections are already in flight behind it.
        if (first) {
            __builtin_amdgcn_s_waitcnt(wait_vm(0));
            __builtin_amdgcn_wave_barrier();
            dma_v(tau);
            first = false;
        } else {
            __builtin_amdgcn_s_waitcnt(wait_vm(VI));
            __builtin_amdgcn_wave_barrier();
        }
        uint8_t* kbuf = wbuf + kb * KB;
        const bool tail_here = appender && tau == tail_tau;
        if (tail_here) {  // the appended record into the LDS copy (word k of record p: chunk-major)
            if (lane < RD) *(uint32_t*)(kbuf + 16 * (64 * (lane >> 2) + tail_p) + 4 * (lane & 3)) = ap_rec;
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_wave_barrier();
        }
        uint32_t rec[RD + 2];
#pragma unroll
        for (int k = 0; k < RD / 4; ++k) {
            const uint4 v4 = *(const uint4*)(kbuf + 16 * (64 * k + qslot));
            rec[4 * k] = v4.x; rec[4 * k + 1] = v4.y; rec[4 * k + 2] = v4.z; rec[4 * k + 3] = v4.w;
        }
        rec[RD] = 0;
        rec[RD + 1] = 0;
        kb ^= 1;
        // 16-bit values: the next K section (into the buffer the previous tile's records
        // left), then the first batch of this tile's value operands, both in flight
        // during QK; loads complete in issue order, so the operands' own waits never
        // wait for the DMA
        u32x4 vr[16];
        if constexpr (V16) {
            if (more) dma_k(tau + kWaves, kb);
            load_v16(tau, IC0{}, IC1{}, vr);
        }
        // ---- QK: this lane's token, 8 fields of one width class per instruction
        floatx16 acc0 = {}, acc1 = {};
        qk_class<8, RD>(sm, rec, cstart[8], cunits[8], cubase[8], qb, acc0, acc1);
        qk_class<7, RD>(sm, rec, cstart[7], cunits[7], cubase[7], qb, acc0, acc1);
        qk_class<6, RD>(sm, rec, cstart[6], cunits[6], cubase[6], qb, acc0, acc1);
        qk_class<5, RD>(sm, rec, cstart[5], cunits[5], cubase[5], qb, acc0, acc1);
        qk_class<4, RD>(sm, rec, cstart[4], cunits[4], cubase[4], qb, acc0, acc1);
        qk_class<3, RD>(sm, rec, cstart[3], cunits[3], cubase[3], qb, acc0, acc1);
        qk_class<2, RD>(sm, rec, cstart[2], cunits[2], cubase[2], qb, acc0, acc1);
        qk_class<1, RD>(sm, rec, cstart[1], cunits[1], cubase[1], qb, acc0, acc1);
        floatx16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = acc0[i] + acc1[i];
        // ---- V section landed (scales, runs); the next K section then goes out (into
        // the K buffer this tile's records left), behind this tile's V in the queue.
        // 16-bit values: the scales landed (the next K section and the first operand
        // batch went out after them), then the second batch goes out
        if constexpr (V16) {
            if (more) __builtin_amdgcn_s_waitcnt(wait_vm(2 * kPre + KI));
            else __builtin_amdgcn_s_waitcnt(wait_vm(2 * kPre));
            __builtin_amdgcn_wave_barrier();
            load_v16(tau, IC1{}, IC2{}, vr);
        } else {
            __builtin_amdgcn_s_waitcnt(wait_vm(0));
            __builtin_amdgcn_wave_barrier();
            if (more) dma_k(tau + kWaves, kb);
        }
        uint8_t* vsec = wbuf + 2 * KB;
        const float* scl = (const float*)(vsec + (V16 ? 0 : VR));
        if constexpr (V16) {
            if (tail_here) {  // the appended scales into the LDS copy (its values: below)
                if (lane == 0) {
                    ((float*)scl)[tail_p] = ap_sk;
                    ((float*)scl)[kTile + tail_p] = ap_sv;
                }
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                __builtin_amdgcn_wave_barrier();
            }
        } else if (tail_here) {  // the appended V codes and scales into the LDS copy
            const int vb = tail_p * V, vk = vb >> 5, vsh = vb & 31;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const uint32_t code = f ? ap_vcq : ap_vcp;
                uint32_t* run = (uint32_t*)vsec + (f ? qq : qp) * 2 * V;
                atomicOr(run + vk, code << vsh);
                if (vsh + V > 32) atomicOr(run + vk + 1, code >> (32 - vsh));
            }
            if (lane == 0) {
                ((float*)scl)[tail_p] = ap_sk;
                ((float*)scl)[kTile + tail_p] = ap_sv;
            }
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_wave_barrier();
        }
        float sk[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 a = *(const float4*)(scl + 16 * grp + 4 * i);
            sk[4 * i] = a.x; sk[4 * i + 1] = a.y; sk[4 * i + 2] = a.z; sk[4 * i + 3] = a.w;
        }
        // ---- logits: hi + lo columns (lanes l and l^8), token scale, ragged-tail mask
        float z[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = (acc[i] + dpp_ror8(acc[i])) * sk[i];
        if (__builtin_expect(nvalid < kTile, 0)) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (16 * grp + i >= nvalid) z[i] = -INFINITY;
        }
        // ---- softmax weights against the lazy reference R = mref + vexp
        float tm = z[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) tm = fmaxf(tm, z[i]);
        tm = xor32_max(xor16_max(tm));
        float sv[16];
        if constexpr (V16) {  // 16-bit values are the values themselves (no norm, no block scale)
#pragma unroll
            for (int i = 0; i < 16; ++i) sv[i] = 1.f;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 b = *(const float4*)(scl + kTile + 16 * grp + 4 * i);
                sv[4 * i] = b.x; sv[4 * i + 1] = b.y; sv[4 * i + 2] = b.z; sv[4 * i + 3] = b.w;
            }
        }
        float smax = sv[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) smax = fmaxf(smax, sv[i]);
        if (__ballot(tm > mref + kRescaleSlack || smax > vlim)) {
            // the tile's largest value norm (all four slot groups) sets the power of two
            const float smx = xor32_max(xor16_max(smax));
            const float vnew = fmaxf(vexp, (float)(__builtin_amdgcn_frexp_expf(smx) - kVNormExp));
            const float mnew = fmaxf(mref, tm);
            const float alpha = __builtin_amdgcn_exp2f((mref + vexp) - (mnew + vnew));
            mref = mnew;
            vexp = vnew;
            vlim = __builtin_amdgcn_ldexpf(1.f, kVNormExp + (int)vnew);
            lrun *= alpha;
            if (lane < 8) sm.alpha[wave][lane] = alpha;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            // PV accumulator row 4*(lane/16) + j holds head (row & 7)
            const float4 al = *(const float4*)&sm.alpha[wave][4 * (grp & 1)];
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                o[ct][0] *= al.x; o[ct][1] *= al.y; o[ct][2] *= al.z; o[ct][3] *= al.w;
            }
            __builtin_amdgcn_wave_barrier();
        }
        const float rref = mref + vexp;
        float psum = 0.f;
        H8 pa[2];
        // hi rows take RZ16(p s^V) and lo rows the binary16 residual p s^V - hi (exact in
        // binary32), so the two rows together carry about 21 bits of each weight
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const float p0 = __builtin_amdgcn_exp2f(z[i] - rref), p1 = __builtin_amdgcn_exp2f(z[i + 1] - rref);
            psum += p0 + p1;
            const float pv0 = p0 * sv[i], pv1 = p1 * sv[i + 1];
            const auto hi = __builtin_amdgcn_cvt_pkrtz(pv0, pv1);
            const float r0 = __builtin_fmaf((float)hi[0], mlo, pv0), r1 = __builtin_fmaf((float)hi[1], mlo, pv1);
            pa[i >> 3].u[(i & 7) >> 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
        }
        lrun += psum;
        // ---- PV: B operand = 16 consecutive slots of coordinate 16*ct + lane%16
        if constexpr (V16) {
            load_v16(tau, IC2{}, IC3{}, vr);
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                H8 b0, b1;
#pragma unroll
                for (int k = 0; k < 4; ++k) { b0.u[k] = vr[2 * ct][k]; b1.u[k] = vr[2 * ct + 1][k]; }
                o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[0].h, b0.h, o[ct], 0, 0, 0);
                o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[1].h, b1.h, o[ct], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const int byte0 = (16 * ct + row) * 8 * V + 2 * V * grp;
                const uint32_t* wv = (const uint32_t*)(vsec + (byte0 & ~3));
                uint32_t vraw[NW + 1];
#pragma unroll
                for (int k = 0; k <= NW; ++k) vraw[k] = wv[k];
                H8 b0, b1;
                decode_v<V>(sm.tab, vraw, (uint32_t)(byte0 & 3) * 8, b0, b1);
                o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[0].h, b0.h, o[ct], 0, 0, 0);
                o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[1].h, b1.h, o[ct], 0, 0, 0);
            }
        }
        // the V buffer is free once its reads have returned
        if (more) {
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_wave_barrier();
            dma_v(tau + kWaves);
        }
    }

    // ---- the appended token into the cache (the tail tile was read from LDS already)
    if (appender) {
        uint8_t* tile = (uint8_t*)head_base + tail_tau * TB;
        if (lane < RD) ((uint32_t*)(tile + tail_p * SK))[lane] = ap_rec;
        uint32_t* vrun = (uint32_t*)(tile + KB);
        const int vb = tail_p * V, vk = vb >> 5, vsh = vb & 31;
#pragma unroll
        for (int f = 0; f < 2 && !V16; ++f) {  // (16-bit values: written in the prologue)
            const uint32_t code = f ? ap_vcq : ap_vcp;
            uint32_t* run = vrun + (f ? qq : qp) * 2 * V;
            if (code != 0) {
                atomicOr(run + vk, code << vsh);
                if (vsh + V > 32 && (code >> (32 - vsh)) != 0) atomicOr(run + vk + 1, code >> (32 - vsh));
            }
        }
        if (lane == 0) {
            float* scl = (float*)(tile + KB + kHeadDim * 8 * V);
            scl[tail_p] = ap_sk;
            scl[kTile + tail_p] = ap_sv;
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
    // each wave's unnormalised output [coordinate][head]: in the wave's own tile buffers
    // when they hold it (its LDS reads of them are behind it, so no barrier first), else
    // in the shared tile buffers once every wave is done with them
    constexpr int kOutBytes = (int)sizeof(float) * kHeadDim * 8;
    constexpr bool kOwnOut = WB >= kOutBytes;
    constexpr int kOutStride = kOwnOut ? WB : kOutBytes;
    static_assert(kWaves * kOutStride <= BUF, "the wave outputs fit the tile buffers");
    if (!kOwnOut) __syncthreads();
    if (lane < 8) { sm.wm[lane][wave] = mref + vexp; sm.wl[lane][wave] = lsum; }
    if (lane < 32) {
        // lane l holds rows 4*(l/16) .. +3 (heads) of coordinates 16*ct + l%16
        float* wo = (float*)(bufs + wave * kOutStride);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
            *(float4*)&wo[(16 * ct + (lane & 15)) * 8 + 4 * (lane >> 4)] = float4{o[ct][0], o[ct][1], o[ct][2], o[ct][3]};
    }
    __syncthreads();
    // merge the four waves: thread (half, c) writes coordinate c of heads 4*half .. 4*half+3
    const int D2 = kHeadDim + 2;
    const int c = tid & (kHeadDim - 1), h0 = 4 * (tid >> 7);
    if (h0 < g) {
        // every LDS read of the combine goes out before any is used
        float4 ow[kWaves], mwj[4], lwj[4];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) ow[w] = *(const float4*)((const float*)(bufs + w * kOutStride) + c * 8 + h0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            mwj[j] = *(const float4*)sm.wm[h0 + j];
            lwj[j] = *(const float4*)sm.wl[h0 + j];
        }
        const float vs = V16 ? 1.f : my_vsig;
        float* const part0 = ws + (((int64_t)s * n_q + kvh * g + h0) * n_split + split) * D2;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int hh = h0 + j;
            if (hh >= g) break;
            const float4 mw = mwj[j];
            const float4 lw = lwj[j];
            const float M = fmaxf(fmaxf(mw.x, mw.y), fmaxf(mw.z, mw.w));
            float l = 0.f, acc = 0.f;
            if (M != -INFINITY) {
                const float f0 = __builtin_amdgcn_exp2f(mw.x - M), f1 = __builtin_amdgcn_exp2f(mw.y - M);
                const float f2 = __builtin_amdgcn_exp2f(mw.z - M), f3 = __builtin_amdgcn_exp2f(mw.w - M);
                l = f0 * lw.x + f1 * lw.y + f2 * lw.z + f3 * lw.w;
                const float o0 = j == 0 ? ow[0].x : j == 1 ? ow[0].y : j == 2 ? ow[0].z : ow[0].w;
                const float o1 = j == 0 ? ow[1].x : j == 1 ? ow[1].y : j == 2 ? ow[1].z : ow[1].w;
                const float o2 = j == 0 ? ow[2].x : j == 1 ? ow[2].y : j == 2 ? ow[2].z : ow[2].w;
                const float o3 = j == 0 ? ow[3].x : j == 1 ? ow[3].y : j == 2 ? ow[3].z : ow[3].w;
                acc = f0 * o0 + f1 * o1 + f2 * o2 + f3 * o3;
            }
            float* part = part0 + (int64_t)j * n_split * D2;
            part[2 + c] = acc * vs;
            if (c == 0) { part[0] = M; part[1] = l; }
        }
    }
}

// launch for one value width V (instantiated in kvq_decode_mfma_v<V>.hip)
template <int V>
hipError_t launch_mfma_v(const kvq_geom& g, const DecodePlan& plan, int n_q_heads, const uint16_t* q,
                         uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len, int n_seq,
                         int64_t max_len, const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                         float scale_log2, float* partials, hipStream_t st, const AppendArgs& app) {
    const int grp = n_q_heads / g.n_kv_heads;
    const int rd = (int)(k_record_bytes(g.k_budget) / 4);
    const int n_chunks = plan.n_split + (app.window > 0 ? window_chunks(app.window) : 0);  // + the window's
    dim3 grid(g.n_kv_heads, n_chunks, n_seq);
#define KVQ_LAUNCH(RDV)                                                                                        \
    if (rd == RDV) {                                                                                            \
        hipLaunchKernelGGL((decode_mfma_kernel<V, RDV>), grid, dim3(256), 0, st, q, cache, seq_byte_off,       \
                           seq_len, max_len, g.capacity_tokens, k_bits, k_sigma, v_sigma, scale_log2, n_q_heads, \
                           grp, g.rope_pairing, g.k_budget, plan.tiles_per_split, n_chunks, partials, app);     \
        return hipGetLastError();                                                                               \
    }
    if constexpr (V <= 8) {
        if (app.k_signs != nullptr) {  // the rotated variant's step (uniform key widths 1..4)
#define KVQ_LAUNCH_ROT(RDV)                                                                                    \
    if (rd == RDV) {                                                                                            \
        hipLaunchKernelGGL((decode_mfma_kernel<V, RDV, true>), grid, dim3(256), 0, st, q, cache, seq_byte_off, \
                           seq_len, max_len, g.capacity_tokens, k_bits, k_sigma, v_sigma, scale_log2, n_q_heads, \
                           grp, g.rope_pairing, g.k_budget, plan.tiles_per_split, n_chunks, partials, app);     \
        return hipGetLastError();                                                                               \
    }
            KVQ_LAUNCH_ROT(4) KVQ_LAUNCH_ROT(8) KVQ_LAUNCH_ROT(12) KVQ_LAUNCH_ROT(16)
#undef KVQ_LAUNCH_ROT
            return hipErrorInvalidValue;
        }
    }
    KVQ_LAUNCH(0) KVQ_LAUNCH(4) KVQ_LAUNCH(8) KVQ_LAUNCH(12) KVQ_LAUNCH(16)
#undef KVQ_LAUNCH
    return hipErrorInvalidValue;
}

// resident workgroups per CU of the instantiation serving geometry g (0 if unknown)
template <int V>
int mfma_blocks_per_cu_v(const kvq_geom& g) {
    const int rd = (int)(k_record_bytes(g.k_budget) / 4);
    int n = 0;
#define KVQ_OCC(RDV)                                                                                         \
    if (rd == RDV) {                                                                                          \
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_mfma_kernel<V, RDV>, 256, 0) != hipSuccess) \
            n = 0;                                                                                            \
        return n;                                                                                             \
    }
    KVQ_OCC(0) KVQ_OCC(4) KVQ_OCC(8) KVQ_OCC(12) KVQ_OCC(16)
#undef KVQ_OCC
    return 0;
}

}  // namespace kvq
