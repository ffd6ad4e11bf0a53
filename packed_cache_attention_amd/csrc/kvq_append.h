// kvq_append.h -- the one-wave append of a token-head into its packed slot, shared by
// the append kernel (kvq_quantize.hip) and the generic decode step's query-table
// launch (kvq_decode_generic.hip).  Quantization and packing as "RoPE-Aware Bit
// Allocation for KV-Cache Quantization" (abstract; Block-GTQ on TQ-MSE) defines them:
// token norm, per-block codes at the allocated widths, records in K order.
#pragma once
#include "kvq_internal.h"

namespace kvq {

// the wave's LDS writes are done and visible to its other lanes (one wave: no s_barrier)
__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Token j of sequence s's run (or the decode step's token), KV head h, by the 64 lanes
// of one wave (lane l: coordinates 2l, 2l+1; block l for the K order).
__device__ __forceinline__ void append_token(
    const uint16_t* __restrict__ kx, const uint16_t* __restrict__ vx, int64_t stride_tok, int64_t stride_head,
    const int64_t* __restrict__ first_slot, const int32_t* __restrict__ n_new, const int64_t* __restrict__ src_row0,
    int max_new, int64_t capacity, const uint8_t* __restrict__ k_bits, const float* __restrict__ k_sigma,
    const float* __restrict__ v_sigma, uint8_t* __restrict__ cache, const int64_t* __restrict__ seq_byte_off,
    int pairing, int k_budget, int v_bits, const int32_t* __restrict__ step_len, const AppendArgs& app, int s, int h,
    int j, int lane) {
#pragma clang fp contract(off)
    const int window = app.window;
    // either explicit runs (first_slot, n_new, src_row0) or the decode step: one token
    // per sequence, row s, into slot step_len[s] - 1; with an fp16 window of `window`
    // tokens, the token leaving it (ring row (step_len[s] - 1) mod window of row s)
    // into slot step_len[s] - window - 1
    const int64_t first = step_len ? (int64_t)step_len[s] - 1 - window : first_slot[s];
    const int n = step_len ? 1 : n_new[s];
    if (first < 0 || n <= 0 || n > max_new || first + n > capacity || j >= n) return;
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
    wave_sync_lds();
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
    wave_sync_lds();
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

}  // namespace kvq
