// kvq_decode_generic.hip -- the vector-ALU decode kernel: packed-cache GQA decode
// attention in binary32 for every geometry the matrix-core kernel does not take (16-bit
// keys or values -- the K-only value mode among them -- key records over 64 bytes, GQA
// groups over 8).  "RoPE-Aware Bit Allocation for KV-Cache Quantization" (abstract):
// the packed-cache serving path reads the compressed cache at decode time.
//
// One wave per 64-token tile, four waves per workgroup, each with its own running
// maximum, weight sums and outputs, combined at the end of the chunk:
//   * logits: lane = token.  The lane stages its K record in LDS (its own column, so
//     every read is conflict-free) and walks the fields in K order -- widths
//     descending, so each width class is one uniform loop -- extracting each code,
//     looking its level up in LDS and multiplying it into the G query heads.  The
//     query values come from a small per-(sequence, KV head) table in the field order
//     with the block scale and softmax scale folded in, read with scalar loads: the
//     multiply-adds take them from scalar registers and the table costs no LDS traffic.
//     The token scale multiplies the finished dot products.
//   * softmax: per head a wave-wide maximum, the weights 2^(z - m), the lane's own
//     running sums; the weights times the token's value norm go to LDS.
//   * values: lane = coordinate c (and c + 64).  The lane holds its two V runs in
//     registers (static bit positions per token), looks each level up and adds
//     weight x level into its outputs for the G heads, the weights read as broadcasts.
// The value block scale multiplies the combined output once.
#include "kvq_internal.h"
#include "kvq_append.h"

namespace kvq {

constexpr int kGenWaves = 4;
constexpr int kGenKRows = 32;  // K record dwords staged at a time (records over 128 bytes are 16-bit: two halves)
constexpr int kGenericQMax = 16;  // query heads per KV head

// query table row (s, kvh): field f of the K order -> G values q_j[c_f] * sigma_(c_f) *
// scale * log2(e) (sigma = 1 for 16-bit keys); heads j >= g hold 0.  One workgroup of
// 256 threads per (KV head, sequence): every load is issued first (the group's queries
// as 8-byte pieces, the widths and scales), the K-order rank of each block comes from
// ballots over the widths, then thread t writes head j's entries for coordinates t, t + 128.
__global__ __launch_bounds__(256) void generic_qtable_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_bits, const float* __restrict__ k_sigma, int n_q,
    int g, int G, int pairing, int k16, float scale_log2, float* __restrict__ table, AppendArgs app,
    const float* __restrict__ v_sigma, uint8_t* __restrict__ cache, const int64_t* __restrict__ seq_byte_off,
    const int32_t* __restrict__ seq_len, int64_t capacity, int k_budget, int v_bits) {
    const int kvh = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
    // the decode step's new token (or the token leaving the fp16 window) for this
    // (sequence, KV head): the last wave packs it, as the append kernel would
    if (app.k != nullptr && tid >= 192)
        append_token(app.k, app.v, app.stride_seq, app.stride_head, nullptr, nullptr, nullptr, 1, capacity, k_bits,
                     k_sigma, v_sigma, cache, seq_byte_off, pairing, k_budget, v_bits, seq_len, app, s, kvh, 0,
                     tid & 63);
    __shared__ float s_q[kGenericQMax][kHeadDim];
    __shared__ int s_pos[kHeadDim];  // coordinate -> field position in the K order (-1: width 0)
    __shared__ float s_sig[kHeadDim];
    const uint16_t* qs = q + ((int64_t)s * n_q + (int64_t)kvh * g) * kHeadDim;
    uint2 qv[kGenericQMax * kHeadDim / 4 / 256];
#pragma unroll
    for (int i = 0; i < kGenericQMax * kHeadDim / 4 / 256; ++i) {
        const int e = 4 * (tid + 256 * i);  // element index in [g][128]
        qv[i] = e < g * kHeadDim ? *(const uint2*)(qs + e) : uint2{0u, 0u};
    }
    const int w = tid < kMaxBlocks ? k_bits[kvh * kMaxBlocks + tid] : 0;
    const float sig = tid < kMaxBlocks ? k_sigma[kvh * kMaxBlocks + tid] : 0.f;
#pragma unroll
    for (int i = 0; i < kGenericQMax * kHeadDim / 4 / 256; ++i) {
        const int e = 4 * (tid + 256 * i);
        if (e < kGenericQMax * kHeadDim) {
            float* d = &s_q[0][0] + e;
            d[0] = h2f(qv[i].x & 0xffffu); d[1] = h2f(qv[i].x >> 16);
            d[2] = h2f(qv[i].y & 0xffffu); d[3] = h2f(qv[i].y >> 16);
        }
    }
    if (tid < kMaxBlocks) {  // wave 0: lane = block; rank by (width desc, index asc)
        const unsigned long long below = (1ull << tid) - 1ull;
        int rank = 0;
        for (int wc = 16; wc >= 1; --wc) {
            const unsigned long long mk = __ballot(w == wc);
            if (wc > w) rank += __popcll(mk);
            if (wc == w) rank += __popcll(mk & below);
        }
        const int cp = pairing == KVQ_PAIR_HALF ? tid : 2 * tid;
        const int cq = pairing == KVQ_PAIR_HALF ? tid + kMaxBlocks : 2 * tid + 1;
        s_pos[cp] = w > 0 ? 2 * rank : -1;
        s_pos[cq] = w > 0 ? 2 * rank + 1 : -1;
        s_sig[cp] = s_sig[cq] = k16 ? 1.f : sig;
    }
    __syncthreads();
    float* t = table + ((int64_t)s * gridDim.x + kvh) * kHeadDim * G;
    for (int e = tid; e < G * kHeadDim; e += 256) {
        const int j = e / kHeadDim, c = e - j * kHeadDim;
        const int f = s_pos[c];
        if (f >= 0) t[f * G + j] = j < g ? s_q[j][c] * s_sig[c] * scale_log2 : 0.f;
    }
}

// fields of width W (n of them, K-order fields f0.., bits off0..) into the G logits
template <int W, int G>
__device__ __forceinline__ void qk_class(const uint32_t* __restrict__ krec, const float* __restrict__ lev,
                                         const float* __restrict__ qt, int n, int f0, int off0, int lane,
                                         float (&z)[G]) {
#pragma unroll 4
    for (int i = 0; i < n; ++i) {
        const int off = off0 + i * W, k = off >> 5, r = off & 31;
        const uint32_t lo = krec[k * 64 + lane], hi = krec[(k + 1) * 64 + lane];
        const uint32_t code = __builtin_amdgcn_alignbit(hi, lo, r) & ((1u << W) - 1u);
        const float lv = lev[KVQ_CB_OFF(W) + code];
        const float* qr = qt + (f0 + i) * G;
#pragma unroll
        for (int j = 0; j < G; ++j) z[j] = fmaf(lv, qr[j], z[j]);
    }
}

// dynamic LDS bytes of one workgroup: levels | per wave K rows | per wave weights,
// reused at the end for the four waves' outputs; at least a window chunk's scratch
__host__ __device__ inline int generic_lds_bytes(int G, int rd, bool window) {
    const int kr = rd < kGenKRows ? rd : kGenKRows;
    const int main_ = 4 * (512 + kGenWaves * (kr + 1) * 64 + kGenWaves * kTile * G);
    const int comb = 4 * (512 + 2 * kGenWaves * G + kGenWaves * G * kHeadDim);
    const int win = window ? 4 * (16 * kHeadDim + 2 * 16 * kWindowChunk) : 0;
    int b = main_ > comb ? main_ : comb;
    return b > win ? b : win;
}

template <int V, int G>
__global__ __launch_bounds__(256) void decode_generic_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, const int64_t* __restrict__ seq_byte_off,
    const int32_t* __restrict__ seq_len, int64_t max_len, int64_t capacity, const uint8_t* __restrict__ k_bits,
    const float* __restrict__ v_sigma, const float* __restrict__ qtab, float scale_log2, int n_q, int g, int pairing,
    int k_budget, int tiles_per_split, int n_split, float* __restrict__ ws, AppendArgs app) {
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    const int split = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (app.window > 0 && split >= n_split - window_chunks(app.window)) {  // the fp16 window's chunks
        window_chunk<16>(app, q, n_q, g, s, kvh, seq_len, scale_log2, ws, n_split,
                         split - (n_split - window_chunks(app.window)), dyn);
        return;
    }
    const int64_t len = min(max((int64_t)seq_len[s] - app.window, (int64_t)0), max_len);
    const int64_t n_tiles_seq = (len + kTile - 1) / kTile;
    const int64_t t0 = (int64_t)split * tiles_per_split;
    const int64_t t1 = min(t0 + tiles_per_split, n_tiles_seq);
    const bool k16 = k_budget == 16 * kMaxBlocks;
    const int SK = (int)k_record_bytes(k_budget), RD = SK / 4;
    const int KR = RD < kGenKRows ? RD : kGenKRows;
    const int64_t TB = tile_bytes(kHeadDim, k_budget, V);
    float* s_lev = dyn;
    uint32_t* krec = (uint32_t*)(dyn + 512) + wave * (KR + 1) * 64;
    float* s_w = dyn + 512 + kGenWaves * (KR + 1) * 64 + wave * kTile * G;
    for (int i = tid; i < 510; i += 256) s_lev[i] = h2f(c_levels[i]);
    // fields per width class (wave-uniform): two per block of that width
    const int my_w = k_bits[kvh * kMaxBlocks + lane];
    int cnt[9];
#pragma unroll
    for (int w = 1; w <= 8; ++w) cnt[w] = 2 * __popcll(__ballot(my_w == w));
    cnt[0] = 0;
    __syncthreads();

    float o0[G], o1[G], lsum[G], m[G];
#pragma unroll
    for (int j = 0; j < G; ++j) { o0[j] = 0.f; o1[j] = 0.f; lsum[j] = 0.f; m[j] = -INFINITY; }
    const float* qt = qtab + ((int64_t)s * gridDim.y + kvh) * kHeadDim * G;
    const uint8_t* head = cache + seq_byte_off[s] + (int64_t)kvh * (capacity / kTile) * TB;
    constexpr int RW = V == 16 ? 32 : 2 * V;  // dwords of one V run

    for (int64_t tau = t0 + wave; tau < t1; tau += kGenWaves) {
        const uint8_t* tile = head + tau * TB;
        const int nvalid = (int)min((int64_t)kTile, len - tau * kTile);
        // this lane's V runs (coordinates lane and lane + 64) and token scales
        uint32_t ra[RW], rb[RW];
        const uint8_t* vsec = tile + kTile * SK;
        if (V == 16) {
#pragma unroll
            for (int i = 0; i < RW / 4; ++i) {
                const uint4 a = ((const uint4*)(vsec + lane * 8 * V))[i];
                const uint4 b = ((const uint4*)(vsec + (lane + 64) * 8 * V))[i];
                ra[4 * i] = a.x; ra[4 * i + 1] = a.y; ra[4 * i + 2] = a.z; ra[4 * i + 3] = a.w;
                rb[4 * i] = b.x; rb[4 * i + 1] = b.y; rb[4 * i + 2] = b.z; rb[4 * i + 3] = b.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < RW / 2; ++i) {
                const uint2 a = ((const uint2*)(vsec + lane * 8 * V))[i];
                const uint2 b = ((const uint2*)(vsec + (lane + 64) * 8 * V))[i];
                ra[2 * i] = a.x; ra[2 * i + 1] = a.y;
                rb[2 * i] = b.x; rb[2 * i + 1] = b.y;
            }
        }
        const float* scl = (const float*)(vsec + kHeadDim * 8 * V);
        const float sk = scl[lane], sv = scl[kTile + lane];

        // ---- logits, lane = token
        float z[G];
#pragma unroll
        for (int j = 0; j < G; ++j) z[j] = 0.f;
        const uint4* rec = (const uint4*)(tile + lane * SK);
        if (k16) {
            // 256-byte records of raw binary16 in block order, staged in two halves
            for (int half = 0; half < 2; ++half) {
#pragma unroll
                for (int i = 0; i < kGenKRows / 4; ++i) {
                    const uint4 x = rec[half * (kGenKRows / 4) + i];
                    krec[(4 * i) * 64 + lane] = x.x;
                    krec[(4 * i + 1) * 64 + lane] = x.y;
                    krec[(4 * i + 2) * 64 + lane] = x.z;
                    krec[(4 * i + 3) * 64 + lane] = x.w;
                }
#pragma unroll 4
                for (int f = 0; f < 2 * kGenKRows; ++f) {
                    const uint32_t wd = krec[(f >> 1) * 64 + lane];
                    const float lv = h2f((f & 1) ? (wd >> 16) : (wd & 0xffffu));
                    const float* qr = qt + (half * 2 * kGenKRows + f) * G;
#pragma unroll
                    for (int j = 0; j < G; ++j) z[j] = fmaf(lv, qr[j], z[j]);
                }
            }
        } else {
            for (int i0 = 0; i0 < RD / 4; i0 += 4) {  // four loads in flight before the first is used
                uint4 x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (i0 + i < RD / 4) x[i] = rec[i0 + i];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i0 + i < RD / 4) {
                        const int k = 4 * (i0 + i);
                        krec[k * 64 + lane] = x[i].x;
                        krec[(k + 1) * 64 + lane] = x[i].y;
                        krec[(k + 2) * 64 + lane] = x[i].z;
                        krec[(k + 3) * 64 + lane] = x[i].w;
                    }
                }
            }
            int f = 0, off = 0;
            qk_class<8, G>(krec, s_lev, qt, cnt[8], f, off, lane, z); f += cnt[8]; off += 8 * cnt[8];
            qk_class<7, G>(krec, s_lev, qt, cnt[7], f, off, lane, z); f += cnt[7]; off += 7 * cnt[7];
            qk_class<6, G>(krec, s_lev, qt, cnt[6], f, off, lane, z); f += cnt[6]; off += 6 * cnt[6];
            qk_class<5, G>(krec, s_lev, qt, cnt[5], f, off, lane, z); f += cnt[5]; off += 5 * cnt[5];
            qk_class<4, G>(krec, s_lev, qt, cnt[4], f, off, lane, z); f += cnt[4]; off += 4 * cnt[4];
            qk_class<3, G>(krec, s_lev, qt, cnt[3], f, off, lane, z); f += cnt[3]; off += 3 * cnt[3];
            qk_class<2, G>(krec, s_lev, qt, cnt[2], f, off, lane, z); f += cnt[2]; off += 2 * cnt[2];
            qk_class<1, G>(krec, s_lev, qt, cnt[1], f, off, lane, z);
        }

        // ---- softmax: running maximum per head, the lane's weight sums, weights to LDS
        const bool valid = lane < nvalid;
        const float ks = k16 ? 1.f : sk, vs = V == 16 ? 1.f : sv;
        float wv[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float zz = valid ? z[j] * ks : -INFINITY;
            const float mn = fmaxf(m[j], wave_max64(zz));
            const float a = exp2f(m[j] - mn);
            const float p = exp2f(zz - mn);
            lsum[j] = lsum[j] * a + p;
            o0[j] *= a;
            o1[j] *= a;
            m[j] = mn;
            wv[j] = p * vs;
        }
#pragma unroll
        for (int j = 0; j < G; j += 4)
            *(float4*)(s_w + lane * G + j) = float4{wv[j], wv[j + 1], wv[j + 2], wv[j + 3]};
        __builtin_amdgcn_wave_barrier();

        // ---- values, lane = coordinate (lane and lane + 64)
#pragma unroll
        for (int p = 0; p < kTile; ++p) {
            float la, lb;
            if (V == 16) {
                const int sh = 16 * (p & 1);
                la = h2f((ra[p >> 1] >> sh) & 0xffffu);
                lb = h2f((rb[p >> 1] >> sh) & 0xffffu);
            } else {
                const int bit = p * V, k = bit >> 5, r = bit & 31;
                const uint32_t ca = (r + V <= 32) ? (ra[k] >> r) : __builtin_amdgcn_alignbit(ra[k + 1], ra[k], r);
                const uint32_t cb = (r + V <= 32) ? (rb[k] >> r) : __builtin_amdgcn_alignbit(rb[k + 1], rb[k], r);
                la = s_lev[KVQ_CB_OFF(V) + (ca & ((1u << V) - 1u))];
                lb = s_lev[KVQ_CB_OFF(V) + (cb & ((1u << V) - 1u))];
            }
            float wp[G];
#pragma unroll
            for (int j = 0; j < G; j += 4) {
                const float4 x = *(const float4*)(s_w + p * G + j);
                wp[j] = x.x; wp[j + 1] = x.y; wp[j + 2] = x.z; wp[j + 3] = x.w;
            }
#pragma unroll
            for (int j = 0; j < G; ++j) {
                o0[j] = fmaf(wp[j], la, o0[j]);
                o1[j] = fmaf(wp[j], lb, o1[j]);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // ---- the four waves' partials combined into the chunk's partial
#pragma unroll
    for (int j = 0; j < G; ++j) lsum[j] = wave_sum64(lsum[j]);
    __syncthreads();  // every wave is done with its staging rows
    float* s_m = dyn + 512;
    float* s_l = s_m + kGenWaves * G;
    float* s_o = s_l + kGenWaves * G;  // [wave][G][128]
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            s_m[wave * G + j] = m[j];
            s_l[wave * G + j] = lsum[j];
        }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
        s_o[(wave * G + j) * kHeadDim + lane] = o0[j];
        s_o[(wave * G + j) * kHeadDim + 64 + lane] = o1[j];
    }
    __syncthreads();
    constexpr int D2 = kHeadDim + 2;
    for (int e = tid; e < g * kHeadDim; e += 256) {
        const int j = e >> 7, c = e & (kHeadDim - 1);
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kGenWaves; ++w) M = fmaxf(M, s_m[w * G + j]);
        float O = 0.f, L = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kGenWaves; ++w) {
                const float f = exp2f(s_m[w * G + j] - M);
                O += f * s_o[(w * G + j) * kHeadDim + c];
                L += f * s_l[w * G + j];
            }
        }
        const int blk = pairing == KVQ_PAIR_HALF ? (c & (kMaxBlocks - 1)) : (c >> 1);
        const float sig = V == 16 ? 1.f : v_sigma[kvh * kMaxBlocks + blk];
        float* part = ws + (((int64_t)s * n_q + (int64_t)kvh * g + j) * n_split + split) * D2;
        part[2 + c] = O * sig;
        if (c == 0) {
            part[0] = M;
            part[1] = L;
        }
    }
}

// ---------------------------------------------------------------- host side
static int generic_G(int grp) { return grp <= 4 ? 4 : (grp <= 8 ? 8 : 16); }

template <int V>
static const void* generic_fn(int G) {
    if (G == 4) return (const void*)decode_generic_kernel<V, 4>;
    if (G == 8) return (const void*)decode_generic_kernel<V, 8>;
    return (const void*)decode_generic_kernel<V, 16>;
}

static const void* generic_kernel_for(int v_bits, int G) {
    switch (v_bits) {
        case 1: return generic_fn<1>(G);
        case 2: return generic_fn<2>(G);
        case 3: return generic_fn<3>(G);
        case 4: return generic_fn<4>(G);
        case 5: return generic_fn<5>(G);
        case 6: return generic_fn<6>(G);
        case 7: return generic_fn<7>(G);
        case 8: return generic_fn<8>(G);
        case 16: return generic_fn<16>(G);
        default: return nullptr;
    }
}

int64_t generic_table_bytes(const kvq_geom& g, int n_q_heads, int n_seq) {
    const int G = generic_G(n_q_heads / g.n_kv_heads);
    return (int64_t)n_seq * g.n_kv_heads * kHeadDim * G * 4;
}

int generic_blocks_per_cu(const kvq_geom& g, int n_q_heads) {
    const int G = generic_G(n_q_heads / g.n_kv_heads);
    const void* fn = generic_kernel_for(g.v_bits, G);
    if (!fn) return 0;
    const int lds = generic_lds_bytes(G, (int)(k_record_bytes(g.k_budget) / 4), false);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 256, lds) != hipSuccess) n = 0;
    return n;
}

hipError_t launch_decode_generic(const kvq_geom& g, int tiles_per_split, int n_chunks, int n_q_heads,
                                 const uint16_t* q, uint8_t* cache, const int64_t* seq_byte_off,
                                 const int32_t* seq_len, int n_seq, int64_t max_len, const uint8_t* k_bits,
                                 const float* k_sigma, const float* v_sigma, float scale_log2, float* partials,
                                 hipStream_t st, const AppendArgs& app) {
    const int grp = n_q_heads / g.n_kv_heads;
    const int G = generic_G(grp);
    // the query table sits after the partials of every chunk
    float* table = partials + (int64_t)n_seq * n_q_heads * n_chunks * (kHeadDim + 2);
    hipLaunchKernelGGL(generic_qtable_kernel, dim3(g.n_kv_heads, n_seq), dim3(256), 0, st, q, k_bits, k_sigma,
                       n_q_heads, grp, G, g.rope_pairing, g.k_budget == 16 * kMaxBlocks ? 1 : 0, scale_log2, table, app,
                       v_sigma, cache, seq_byte_off, seq_len, g.capacity_tokens, g.k_budget, g.v_bits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int lds = generic_lds_bytes(G, (int)(k_record_bytes(g.k_budget) / 4), app.window > 0);
    dim3 grid(n_chunks, g.n_kv_heads, n_seq);
#define KVQ_GEN(VV, GG)                                                                                          \
    if (g.v_bits == VV && G == GG) {                                                                             \
        hipLaunchKernelGGL((decode_generic_kernel<VV, GG>), grid, dim3(256), lds, st, q, cache, seq_byte_off,    \
                           seq_len, max_len, g.capacity_tokens, k_bits, v_sigma, table, scale_log2, n_q_heads, grp, \
                           g.rope_pairing, g.k_budget, tiles_per_split, n_chunks, partials, app);               \
        return hipGetLastError();                                                                                \
    }
#define KVQ_GEN_V(VV) KVQ_GEN(VV, 4) KVQ_GEN(VV, 8) KVQ_GEN(VV, 16)
    KVQ_GEN_V(1) KVQ_GEN_V(2) KVQ_GEN_V(3) KVQ_GEN_V(4) KVQ_GEN_V(5) KVQ_GEN_V(6) KVQ_GEN_V(7) KVQ_GEN_V(8)
    KVQ_GEN_V(16)
#undef KVQ_GEN_V
#undef KVQ_GEN
    return hipErrorInvalidValue;
}

}  // namespace kvq
