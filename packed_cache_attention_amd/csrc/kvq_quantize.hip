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

__global__ __launch_bounds__(256) void quantize_pack_kernel(
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

    const int64_t SK = k_record_bytes(k_budget);
    const int64_t TB = tile_bytes(kHeadDim, k_budget, v_bits);
    const int64_t n_tiles = capacity / kTile;
    uint8_t* tile = cache + seq_byte_off[s] + ((int64_t)h * n_tiles + tau) * TB;

    __shared__ uint16_t s_kc[kTile][kHeadDim];
    __shared__ uint16_t s_vc[kTile][kHeadDim];
    __shared__ float s_ks[kTile], s_vs[kTile];
    __shared__ uint8_t s_w[kHeadDim];          // key width per coordinate
    __shared__ float s_ksig[kHeadDim], s_vsig[kHeadDim];
    __shared__ uint8_t s_fc[kHeadDim];         // K order: coordinate of field f
    __shared__ uint16_t s_fo[kHeadDim];        // bit offset of field f in the record
    __shared__ uint8_t s_fw[kHeadDim];         // width of field f
    __shared__ uint8_t s_first[64];            // first field touching record dword k
    __shared__ int s_nf;
    __shared__ float s_thr[510];               // the codebook thresholds, staged once

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // ---- phase 0: per-head tables and the K order ----
    for (int i = tid; i < 510; i += 256) s_thr[i] = c_thresholds[i];
    if (tid < kMaxBlocks) {
        // rank blocks by (width desc, index asc) with wave ballots; offsets are prefix
        // sums of 2*width in that order
        const int i = tid;
        const int w = k_bits[h * kMaxBlocks + i];
        const int p = pairing == KVQ_PAIR_HALF ? i : 2 * i;
        const int q = pairing == KVQ_PAIR_HALF ? i + kMaxBlocks : 2 * i + 1;
        s_w[p] = s_w[q] = (uint8_t)w;
        s_ksig[p] = s_ksig[q] = k_sigma[h * kMaxBlocks + i];
        s_vsig[p] = s_vsig[q] = v_sigma[h * kMaxBlocks + i];
        const unsigned long long below = (1ull << i) - 1ull;
        int rank = 0, off = 0;
        for (int wc = 16; wc >= 1; --wc) {
            const unsigned long long mk = __ballot(w == wc);
            if (wc > w) { rank += __popcll(mk); off += 2 * wc * __popcll(mk); }
            if (wc == w) { rank += __popcll(mk & below); off += 2 * wc * __popcll(mk & below); }
        }
        if (w > 0) {
            s_fc[2 * rank] = (uint8_t)p; s_fo[2 * rank] = (uint16_t)off; s_fw[2 * rank] = (uint8_t)w;
            s_fc[2 * rank + 1] = (uint8_t)q; s_fo[2 * rank + 1] = (uint16_t)(off + w); s_fw[2 * rank + 1] = (uint8_t)w;
        }
        const unsigned long long nz = __ballot(w > 0);
        if (i == 0) s_nf = 2 * __popcll(nz);
    }
    __syncthreads();
    const int nf = s_nf;
    if (tid < (int)(SK / 4)) {
        int f = 0;
        while (f < nf && s_fo[f] + s_fw[f] <= 32 * tid) ++f;
        s_first[tid] = (uint8_t)f;
    }

    // ---- phase 1: codes ----
    for (int64_t slot = lo_slot + wave; slot < hi_slot; slot += 4) {
        const int p = (int)(slot - tile0);
        const int64_t row = src_row0[s] + (slot - first);
        const uint32_t kp = *(const uint32_t*)(kx + row * stride_tok + (int64_t)h * stride_head + 2 * lane);
        const uint32_t vp = *(const uint32_t*)(vx + row * stride_tok + (int64_t)h * stride_head + 2 * lane);
        const float sk = token_norm(kp), sv = token_norm(vp);
        const int c0 = 2 * lane, c1 = 2 * lane + 1;
        s_kc[p][c0] = (uint16_t)encode(s_thr, kp & 0xffffu, s_w[c0], s_ksig[c0], sk);
        s_kc[p][c1] = (uint16_t)encode(s_thr, kp >> 16, s_w[c1], s_ksig[c1], sk);
        s_vc[p][c0] = (uint16_t)encode(s_thr, vp & 0xffffu, v_bits, s_vsig[c0], sv);
        s_vc[p][c1] = (uint16_t)encode(s_thr, vp >> 16, v_bits, s_vsig[c1], sv);
        if (lane == 0) { s_ks[p] = sk; s_vs[p] = sv; }
    }
    __syncthreads();

    // ---- phase 2: assemble the tile ----
    const int lo_p = (int)(lo_slot - tile0), hi_p = (int)(hi_slot - tile0);
    const bool whole = lo_p == 0 && hi_p == kTile;
    // K records (each belongs to one slot: plain stores)
    const int skd = (int)(SK / 4);
    uint32_t* krec = (uint32_t*)tile;
    for (int idx = tid; idx < kTile * skd; idx += 256) {
        const int p = idx / skd, k = idx - p * skd;
        if (p < lo_p || p >= hi_p) continue;
        uint32_t val = 0;
        const int lo_bit = 32 * k;
        for (int f = s_first[k]; f < nf && s_fo[f] < lo_bit + 32; ++f) {
            const uint32_t code = s_kc[p][s_fc[f]];
            const int sh = (int)s_fo[f] - lo_bit;
            val |= sh >= 0 ? (code << sh) : (code >> (-sh));
        }
        krec[idx] = val;
    }
    // V runs (shared by slots: read-modify-write unless the whole tile is new)
    const int vd = 2 * v_bits;
    uint32_t* vrun = (uint32_t*)(tile + kTile * SK);
    for (int idx = tid; idx < kHeadDim * vd; idx += 256) {
        const int c = idx / vd, k = idx - c * vd;
        const int lo_bit = 32 * k;
        const int pa = max(lo_bit / v_bits, lo_p);
        const int pb = min((lo_bit + 31) / v_bits, hi_p - 1);
        uint32_t val = 0;
        for (int p = pa; p <= pb; ++p) {
            const uint32_t code = s_vc[p][c];
            const int sh = p * v_bits - lo_bit;
            val |= sh >= 0 ? (code << sh) : (code >> (-sh));
        }
        if (whole) vrun[idx] = val;
        else if (pa <= pb) vrun[idx] |= val;
    }
    // scales
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
    hipLaunchKernelGGL(quantize_pack_kernel, grid, dim3(256), 0, st, k, v, stride_tok, stride_head, first_slot,
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
