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
// by 64 lanes touches distinct banks).  Norms: waves 0-1 form the two 64-leaf
// halves of each K row's pairwise tree, waves 2-3 those of V (the root adds the
// halves, as the tree does).  Codes: each wave takes a run of K-order fields
// holding about a quarter of the record's bits, and a quarter of the V
// coordinates; for a field every lane searches at the same width, and the K record
// bits are gathered in registers and OR-ed into the LDS records word by word.
constexpr int kRowDw = kHeadDim / 2 + 1;
typedef __attribute__((address_space(3))) const float lds_cf32;  // LDS pointer (32-bit addresses)
__device__ __forceinline__ uint32_t lds_off(lds_cf32* p) { return (uint32_t)(uintptr_t)p; }
constexpr int kQWaves = 8;  // waves per workgroup
constexpr int kQThreads = 64 * kQWaves;
constexpr int kGroup = 4;   // K fields encoded side by side (independent searches)
constexpr int kVGroup = 8;  // V coordinates encoded side by side

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
    const int RW = (int)(SK / 4), RS = RW + 1;  // record words, LDS record stride (odd)
    const int VW = 2 * v_bits, VS = VW + 1;     // run words, LDS run stride
    uint8_t* tile = cache + seq_byte_off[s] + ((int64_t)h * (capacity / kTile) + tau) * TB;

    __shared__ uint32_t s_k[kTile * kRowDw], s_v[kTile * kRowDw];
    __shared__ float s_thr[510];
    __shared__ float s_quarter[kQWaves][kTile];
    __shared__ float s_ks[kTile], s_vs[kTile];
    // K order, field f: x = coordinate | width << 7 | bit offset << 12 | (later fields of
    // the same width) << 23, y = the block's sigma bits; padded so that reads of up to
    // kGroup fields from any f stay in the array
    __shared__ uint2 s_meta[kHeadDim + kGroup];
    __shared__ float s_vsig[kHeadDim];
    __shared__ int s_range[kQWaves + 1];                  // wave w encodes fields [s_range[w], s_range[w+1])
    extern __shared__ uint32_t s_dyn[];                  // records [64][RS], then runs [128][VS]
    uint32_t* s_rec = s_dyn;
    uint32_t* s_run = s_dyn + kTile * RS;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // ---- phase 0: rows, thresholds, K order, zeroed records and runs
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
    for (int i = tid; i < kTile * RS + kHeadDim * VS; i += kQThreads) s_dyn[i] = 0u;
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
        int rank = 0, off = 0, after = 0;
        for (int wc = 16; wc >= 1; --wc) {
            const unsigned long long mk = __ballot(w == wc);
            if (wc > w) { rank += __popcll(mk); off += 2 * wc * __popcll(mk); }
            if (wc == w) {
                rank += __popcll(mk & below);
                off += 2 * wc * __popcll(mk & below);
                after = __popcll(mk & ~below) - 1;  // same-width blocks ranked after this one
            }
        }
        const int nf = 2 * __popcll(__ballot(w > 0));
        if (w > 0) {
            const int pc = pairing == KVQ_PAIR_HALF ? i : 2 * i;
            const int qc = pairing == KVQ_PAIR_HALF ? i + kMaxBlocks : 2 * i + 1;
            const uint32_t sb = __float_as_uint(sig);
            s_meta[2 * rank] = make_uint2(pc | w << 7 | off << 12 | (2 * after + 1) << 23, sb);
            s_meta[2 * rank + 1] = make_uint2(qc | w << 7 | (off + w) << 12 | (2 * after) << 23, sb);
        }
        if (i < kGroup) s_meta[kHeadDim + i] = make_uint2(0u, 0u);
        // split the fields into four runs of about a quarter of the record's bits each
        int wsum = w;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) wsum += __shfl_xor(wsum, m);
        const int total = 2 * wsum;
        // the field at rank 2r starts at `off`; run w starts at the first field whose
        // offset reaches w/4 of the total (offsets increase with rank)
        for (int wv = 0; wv <= kQWaves; ++wv) {
            const int bound = (int)(((int64_t)total * wv + kQWaves - 1) / kQWaves);
            const unsigned long long before = __ballot(w > 0 && off < bound);
            // fields before the bound: 2 per block that starts before it, minus a q
            // field that already starts past it
            const unsigned long long qpast = __ballot(w > 0 && off < bound && off + w >= bound);
            if (i == 0) s_range[wv] = wv == kQWaves ? nf : 2 * __popcll(before) - __popcll(qpast);
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

    // ---- phase 2: codes (lane = token), K record bits gathered per word
    const bool valid = lane >= lo_p && lane < hi_p;
    {
        const float sk = s_ks[lane];
        const uint16_t* krow = (const uint16_t*)(s_k + lane * kRowDw);
        // the field tables are the same for every lane: keep them in scalar registers
        const int f0 = __builtin_amdgcn_readfirstlane(s_range[wave]);
        const int f1 = __builtin_amdgcn_readfirstlane(s_range[wave + 1]);
        int cur = f0 < f1 ? (int)((__builtin_amdgcn_readfirstlane(s_meta[f0].x) >> 12) & 2047) >> 5 : 0;
        uint32_t acc = 0u, nxt = 0u;
        for (int f = f0; f < f1;) {
            // up to kGroup fields of one width (the K order sorts by width) searched side by side
            uint32_t mx[kGroup];
            float sg[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                const uint2 m = s_meta[f + i];
                mx[i] = __builtin_amdgcn_readfirstlane(m.x);
                sg[i] = __uint_as_float(__builtin_amdgcn_readfirstlane(m.y));
            }
            const int wf = (mx[0] >> 7) & 31;
            const int gn = min(min(kGroup, (int)(mx[0] >> 23) + 1), f1 - f);
            uint32_t code[kGroup];
            if (wf == 16) {
#pragma unroll
                for (int i = 0; i < kGroup; ++i) code[i] = krow[mx[i] & 127];
            } else {
                // binary lifting on threshold addresses: t[i] points at the largest
                // threshold found so far that the value reaches (the code's entry)
                lds_cf32* thr = (lds_cf32*)(s_thr + KVQ_CB_OFF(wf));
                float x[kGroup];
                lds_cf32* t[kGroup];
#pragma unroll
                for (int i = 0; i < kGroup; ++i) {
                    x[i] = h2f(krow[mx[i] & 127]);
                    t[i] = thr;
                }
                for (int bit = 1 << (wf - 1); bit >= 1; bit >>= 1) {
                    lds_cf32* c[kGroup];
                    float a[kGroup];
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) {
                        c[i] = t[i] + bit;
                        a[i] = *c[i];
                    }
#pragma unroll
                    for (int i = 0; i < kGroup; ++i) {
                        const float b = sk * (sg[i] * a[i]);
                        if (x[i] >= b) t[i] = c[i];
                    }
                }
#pragma unroll
                for (int i = 0; i < kGroup; ++i) code[i] = (lds_off(t[i]) - lds_off(thr)) >> 2;
            }
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                if (i < gn) {
                    const int of = (mx[i] >> 12) & 2047;
                    const int k = of >> 5, sh = of & 31;
                    if (k != cur) {  // fields are consecutive in bits: the window moves by one word
                        if (valid && acc) atomicOr(&s_rec[lane * RS + cur], acc);
                        acc = nxt;
                        nxt = 0u;
                        cur = k;
                    }
                    acc |= code[i] << sh;
                    if (sh + wf > 32) nxt |= code[i] >> (32 - sh);
                }
            }
            f += gn;
        }
        if (valid && acc) atomicOr(&s_rec[lane * RS + cur], acc);
        if (valid && nxt) atomicOr(&s_rec[lane * RS + cur + 1], nxt);

        const float sv = s_vs[lane];
        const uint16_t* vrow = (const uint16_t*)(s_v + lane * kRowDw);
        const int bit0 = lane * v_bits, vk = bit0 >> 5, vsh = bit0 & 31;
        lds_cf32* vthr = (lds_cf32*)(s_thr + KVQ_CB_OFF(v_bits));
        constexpr int kVPer = kHeadDim / kQWaves;  // V coordinates per wave
        // codes of G consecutive tokens (G * v_bits <= 32, G <= 16) are OR-ed across
        // lanes into the group's first lane before the LDS update, so few lanes share a
        // run word in one atomic
        const int lg = v_bits == 1 ? 4 : v_bits == 2 ? 4 : v_bits <= 4 ? 3 : v_bits <= 8 ? 2 : 1;
        const int G = 1 << lg;
        const int gbits = G * v_bits;
        for (int c0 = kVPer * wave; c0 < kVPer * wave + kVPer; c0 += kVGroup) {
            uint32_t code[kVGroup];
            if (v_bits == 16) {
#pragma unroll
                for (int i = 0; i < kVGroup; ++i) code[i] = vrow[c0 + i];
            } else {
                float x[kVGroup], sg[kVGroup];
                lds_cf32* t[kVGroup];
#pragma unroll
                for (int i = 0; i < kVGroup; ++i) {
                    x[i] = h2f(vrow[c0 + i]);
                    sg[i] = s_vsig[c0 + i];
                    t[i] = vthr;
                }
                for (int bit = 1 << (v_bits - 1); bit >= 1; bit >>= 1) {
                    lds_cf32* c[kVGroup];
                    float a[kVGroup];
#pragma unroll
                    for (int i = 0; i < kVGroup; ++i) {
                        c[i] = t[i] + bit;
                        a[i] = *c[i];
                    }
#pragma unroll
                    for (int i = 0; i < kVGroup; ++i) {
                        const float b = sv * (sg[i] * a[i]);
                        if (x[i] >= b) t[i] = c[i];
                    }
                }
#pragma unroll
                for (int i = 0; i < kVGroup; ++i) code[i] = (lds_off(t[i]) - lds_off(vthr)) >> 2;
            }
#pragma unroll
            for (int i = 0; i < kVGroup; ++i) {
                uint32_t u = valid ? code[i] : 0u;
                u |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x101, 0xf, 0xf, true) << v_bits;
                if (lg >= 2) u |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x102, 0xf, 0xf, true) << (2 * v_bits);
                if (lg >= 3) u |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x104, 0xf, 0xf, true) << (4 * v_bits);
                if (lg >= 4) u |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x108, 0xf, 0xf, true) << (8 * v_bits);
                if (gbits < 32) u &= (1u << gbits) - 1u;
                if ((lane & (G - 1)) == 0 && u) {
                    atomicOr(&s_run[(c0 + i) * VS + vk], u << vsh);
                    if (vsh + gbits > 32) atomicOr(&s_run[(c0 + i) * VS + vk + 1], u >> (32 - vsh));
                }
            }
        }
    }
    __syncthreads();

    // ---- phase 3: the tile's records (valid slots), runs and scales
    uint32_t* krec = (uint32_t*)tile;
    for (int idx = tid; idx < kTile * RW; idx += kQThreads) {
        const int p = idx / RW, k = idx - p * RW;
        if (p >= lo_p && p < hi_p) krec[idx] = s_rec[p * RS + k];
    }
    const bool whole = lo_p == 0 && hi_p == kTile;
    uint32_t* vrun = (uint32_t*)(tile + kTile * SK);
    for (int idx = tid; idx < kHeadDim * VW; idx += kQThreads) {
        const int c = idx / VW, k = idx - c * VW;
        const uint32_t val = s_run[c * VS + k];
        if (whole) vrun[idx] = val;
        else if (val) vrun[idx] |= val;
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
    int pairing, int k_budget, int v_bits, const int32_t* __restrict__ step_len) {
    const int s = blockIdx.z, h = blockIdx.y, j = blockIdx.x;
    // either explicit runs (first_slot, n_new, src_row0) or the decode step: one token
    // per sequence, row s, into slot step_len[s] - 1
    const int64_t first = step_len ? (int64_t)step_len[s] - 1 : first_slot[s];
    const int n = step_len ? 1 : n_new[s];
    if (first < 0 || n <= 0 || n > max_new || first + n > capacity || j >= n) return;
    const int lane = threadIdx.x;
    const int64_t slot = first + j;
    const int64_t row = step_len ? (int64_t)s : src_row0[s] + j;
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
    const uint32_t kp = *(const uint32_t*)(kx + row * stride_tok + (int64_t)h * stride_head + c0);
    const uint32_t vp = *(const uint32_t*)(vx + row * stride_tok + (int64_t)h * stride_head + c0);
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
}

hipError_t launch_quantize_pack(const kvq_geom& g, const uint16_t* k, const uint16_t* v, int64_t stride_tok,
                                int64_t stride_head, int n_seq, const int64_t* first_slot, const int32_t* n_new,
                                const int64_t* src_row0, int max_new, const uint8_t* k_bits, const float* k_sigma,
                                const float* v_sigma, uint8_t* cache, const int64_t* seq_byte_off, hipStream_t st) {
    if (max_new <= kAppendMax) {
        dim3 grid(max_new, g.n_kv_heads, n_seq);
        hipLaunchKernelGGL(append_kernel, grid, dim3(64), 0, st, k, v, stride_tok, stride_head, first_slot, n_new,
                           src_row0, max_new, g.capacity_tokens, k_bits, k_sigma, v_sigma, cache, seq_byte_off,
                           g.rope_pairing, g.k_budget, g.v_bits, (const int32_t*)nullptr);
        return hipGetLastError();
    }
    // a run of max_new slots starting anywhere touches at most ceil(max_new/64) + 1 tiles
    const int tiles = (max_new + kTile - 1) / kTile + 1;
    dim3 grid(tiles, g.n_kv_heads, n_seq);
    // records [64][words + 1] and runs [128][2 v_bits + 1] in dynamic LDS; beside the
    // ~38 KB of static LDS the widest geometry (raw K, 16-bit V) needs ~72 KB per
    // workgroup, which gfx950's 160 KB LDS holds once the launch limit is raised
    const size_t dyn = (size_t)4 * (kTile * (k_record_bytes(g.k_budget) / 4 + 1) + kHeadDim * (2 * g.v_bits + 1));
    static size_t dyn_set = 0;
    if (dyn > dyn_set && dyn > 16384) {
        const hipError_t e = hipFuncSetAttribute((const void*)quantize_pack_kernel,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
        if (e != hipSuccess) return e;
        dyn_set = dyn;
    }
    hipLaunchKernelGGL(quantize_pack_kernel, grid, dim3(kQThreads), dyn, st, k, v, stride_tok, stride_head, first_slot,
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
                       g.v_bits, seq_len);
    return hipGetLastError();
}

}  // namespace kvq
