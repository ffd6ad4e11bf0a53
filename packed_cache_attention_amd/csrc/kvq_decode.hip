// kvq_decode.hip -- packed-cache GQA decode attention, split over the token axis,
// plus the log-sum-exp merge of the split partials.  The page "RoPE-Aware Bit
// Allocation for KV-Cache Quantization" (abstract) describes a packed-cache
// serving path that reads the compressed cache at decode time; this file holds
// the generic (VALU + LDS) kernel that serves every width, including 16-bit
// passthrough, and the merge shared with the matrix-core kernel.
//
// Partials: workspace[((s*n_q + hq)*n_split + split)*(d+2) + {0: m, 1: l, 2+c: o_c}],
// with m in log2 units (logits are pre-multiplied by log2 e) and o unnormalised.
#include <math.h>

#include <algorithm>

#include "kvq_internal.h"

namespace kvq {

constexpr int kGenericMaxGroup = 16;
constexpr bool kMfmaKernel = true;

// bits [pos, pos + w) of a little-endian bitstream at base (w <= 16); reads only
// the (aligned) dwords that hold the field
__device__ __forceinline__ uint32_t read_field(const uint8_t* base, int pos, int w) {
    const uint32_t* dw = (const uint32_t*)base;
    const int k = pos >> 5, sh = pos & 31;
    uint32_t v = dw[k] >> sh;
    if (sh + w > 32) v |= dw[k + 1] << (32 - sh);
    return v & ((1u << w) - 1u);
}

__device__ __forceinline__ float level(uint32_t code, int w) {
    if (w == 16) return h2f(code);
    return h2f(c_levels[min(KVQ_CB_OFF(w) + (int)code, 509)]);
}

// grid: (n_split, n_kv, n_seq); block: 256 threads
__global__ __launch_bounds__(256) void decode_generic_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, const int64_t* __restrict__ seq_byte_off,
    const int32_t* __restrict__ seq_len, int64_t max_len, int64_t capacity, const uint8_t* __restrict__ k_bits,
    const float* __restrict__ k_sigma, const float* __restrict__ v_sigma, float scale_log2, int n_q, int g,
    int pairing, int k_budget, int v_bits, int tiles_per_split, int n_split, float* __restrict__ ws, int len_sub) {
    const int split = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x;
    // packed tokens (seq_len less the fp16 window, if any)
    const int64_t len = min(max((int64_t)seq_len[s] - len_sub, (int64_t)0), max_len);
    const int64_t n_tiles_seq = (len + kTile - 1) / kTile;
    const int64_t t0 = (int64_t)split * tiles_per_split;
    const int64_t t1 = min(t0 + tiles_per_split, n_tiles_seq);
    const int D2 = kHeadDim + 2;

    __shared__ float s_x[kTile][kHeadDim + 1];  // dequantized K, then V, of the current tile
    __shared__ float s_q[kGenericMaxGroup][kHeadDim];
    __shared__ float s_p[kGenericMaxGroup][kTile];
    __shared__ float s_m[kGenericMaxGroup], s_l[kGenericMaxGroup], s_a[kGenericMaxGroup];
    __shared__ float s_ksig[kHeadDim], s_vsig[kHeadDim];
    __shared__ uint8_t s_bw[kMaxBlocks];
    __shared__ uint8_t s_fc[kHeadDim], s_fw[kHeadDim];
    __shared__ uint16_t s_fo[kHeadDim];
    __shared__ int s_nf;

    // per-(KV head) tables: block scales per coordinate and the K order
    if (tid < kMaxBlocks) {
        const int i = tid;
        const int p = pairing == KVQ_PAIR_HALF ? i : 2 * i;
        const int qq = pairing == KVQ_PAIR_HALF ? i + kMaxBlocks : 2 * i + 1;
        s_bw[i] = k_bits[kvh * kMaxBlocks + i];
        s_ksig[p] = s_ksig[qq] = k_sigma[kvh * kMaxBlocks + i];
        s_vsig[p] = s_vsig[qq] = v_sigma[kvh * kMaxBlocks + i];
    }
    for (int idx = tid; idx < g * kHeadDim; idx += 256) {
        const int j = idx / kHeadDim, c = idx - j * kHeadDim;
        s_q[j][c] = h2f(q[((int64_t)s * n_q + kvh * g + j) * kHeadDim + c]);
    }
    if (tid < g) { s_m[tid] = -INFINITY; s_l[tid] = 0.f; }
    __syncthreads();
    if (tid < kMaxBlocks) {
        const int i = tid, w = s_bw[i];
        int rank = 0, off = 0;
        for (int j = 0; j < kMaxBlocks; ++j) {
            const int wj = s_bw[j];
            if (wj > w || (wj == w && j < i)) { ++rank; off += 2 * wj; }
        }
        if (w > 0) {
            const int p = pairing == KVQ_PAIR_HALF ? i : 2 * i;
            const int qq = pairing == KVQ_PAIR_HALF ? i + kMaxBlocks : 2 * i + 1;
            s_fc[2 * rank] = (uint8_t)p; s_fo[2 * rank] = (uint16_t)off; s_fw[2 * rank] = (uint8_t)w;
            s_fc[2 * rank + 1] = (uint8_t)qq; s_fo[2 * rank + 1] = (uint16_t)(off + w); s_fw[2 * rank + 1] = (uint8_t)w;
        }
        const unsigned long long nz = __ballot(w > 0);
        if (i == 0) s_nf = 2 * __popcll(nz);
    }
    __syncthreads();
    const int nf = s_nf;

    const int64_t SK = k_record_bytes(k_budget);
    const int64_t TB = tile_bytes(kHeadDim, k_budget, v_bits);
    const uint8_t* head = cache + seq_byte_off[s] + (int64_t)kvh * (capacity / kTile) * TB;
    const int per = (g * kHeadDim + 255) / 256;  // (head, coordinate) outputs per thread
    float o[kGenericMaxGroup * kHeadDim / 256];
    for (int r = 0; r < per; ++r) o[r] = 0.f;

    for (int64_t tau = t0; tau < t1; ++tau) {
        const uint8_t* tile = head + tau * TB;
        const float* scl = (const float*)(tile + kTile * SK + kHeadDim * 8 * v_bits);
        const int nvalid = (int)min((int64_t)kTile, len - tau * kTile);
        // dequantize K (width-0 coordinates are 0)
        for (int idx = tid; idx < kTile * (kHeadDim + 1); idx += 256) (&s_x[0][0])[idx] = 0.f;
        __syncthreads();
        for (int idx = tid; idx < kTile * nf; idx += 256) {
            const int p = idx / nf, f = idx - p * nf;
            const int w = s_fw[f], c = s_fc[f];
            const uint32_t code = read_field(tile + p * SK, s_fo[f], w);
            const float lv = level(code, w);
            s_x[p][c] = w == 16 ? lv : scl[p] * s_ksig[c] * lv;
        }
        __syncthreads();
        // logits (log2 units); padding slots of a ragged last tile are masked
        for (int idx = tid; idx < g * kTile; idx += 256) {
            const int j = idx / kTile, p = idx - j * kTile;
            float z = 0.f;
            for (int c = 0; c < kHeadDim; ++c) z += s_q[j][c] * s_x[p][c];
            s_p[j][p] = p < nvalid ? z * scale_log2 : -INFINITY;
        }
        __syncthreads();
        // online softmax, one thread per head
        if (tid < g) {
            const int j = tid;
            float mt = -INFINITY;
            for (int p = 0; p < kTile; ++p) mt = fmaxf(mt, s_p[j][p]);
            const float mn = fmaxf(s_m[j], mt);
            const float a = exp2f(s_m[j] - mn);
            float l = 0.f;
            for (int p = 0; p < kTile; ++p) {
                const float e = exp2f(s_p[j][p] - mn);
                s_p[j][p] = e;
                l += e;
            }
            s_l[j] = s_l[j] * a + l;
            s_m[j] = mn;
            s_a[j] = a;
        }
        __syncthreads();
        // dequantize V
        for (int idx = tid; idx < kTile * kHeadDim; idx += 256) {
            const int c = idx / kTile, p = idx - c * kTile;
            const uint32_t code = read_field(tile + kTile * SK + c * 8 * v_bits, p * v_bits, v_bits);
            const float lv = level(code, v_bits);
            s_x[p][c] = v_bits == 16 ? lv : scl[kTile + p] * s_vsig[c] * lv;
        }
        __syncthreads();
        for (int r = 0; r < per; ++r) {
            const int idx = tid + 256 * r;
            if (idx >= g * kHeadDim) break;
            const int j = idx / kHeadDim, c = idx - j * kHeadDim;
            float acc = o[r] * s_a[j];
            for (int p = 0; p < kTile; ++p) acc += s_p[j][p] * s_x[p][c];
            o[r] = acc;
        }
        __syncthreads();
    }
    // partials (an empty chunk writes m = -inf, l = 0, o = 0)
    for (int r = 0; r < per; ++r) {
        const int idx = tid + 256 * r;
        if (idx >= g * kHeadDim) break;
        const int j = idx / kHeadDim, c = idx - j * kHeadDim;
        float* part = ws + (((int64_t)s * n_q + kvh * g + j) * n_split + split) * D2;
        part[2 + c] = o[r];
        if (c == 0) { part[0] = s_m[j]; part[1] = s_l[j]; }
    }
}

// grid: n_seq * n_q rows; block: 256 threads = 2 split halves x 128 coordinates
// Split merge: out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j.  A workgroup
// takes 32 coordinates of one row; its 32 split groups stride over the splits with
// their own running maximum, eight splits' loads in flight at a time, and are
// combined through LDS at the end.
constexpr int kMergeCols = 32, kMergeGroups = 32, kMergeUnroll = 8;

__global__ __launch_bounds__(kMergeCols * kMergeGroups) void merge_kernel(const float* __restrict__ ws, int n_split,
                                                                           float* __restrict__ out) {
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, sg = tid / kMergeCols, c = blockIdx.y * kMergeCols + tid % kMergeCols;
    constexpr int D2 = kHeadDim + 2;
    const float* part = ws + row * n_split * D2;
    float M = -INFINITY, L = 0.f, A = 0.f;
    for (int sp0 = sg; sp0 < n_split; sp0 += kMergeGroups * kMergeUnroll) {
        float m[kMergeUnroll], l[kMergeUnroll], o[kMergeUnroll];
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const int sp = sp0 + u * kMergeGroups;
            const float* p = part + (int64_t)min(sp, n_split - 1) * D2;
            m[u] = sp < n_split ? p[0] : -INFINITY;
            l[u] = p[1];
            o[u] = p[2 + c];
        }
        float mx = M;
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) mx = fmaxf(mx, m[u]);
        if (mx == -INFINITY) continue;  // nothing attended yet in these splits
        const float r = exp2f(M - mx);
        L *= r;
        A *= r;
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const float a = exp2f(m[u] - mx);
            L += a * l[u];
            A += a * o[u];
        }
        M = mx;
    }
    // the wave's two split groups (lanes l and l ^ 32 share a column) first, then the
    // 16 waves' results through LDS, each half of wave 0 taking eight of them
    {
        const float oM = __shfl_xor(M, 32), oL = __shfl_xor(L, 32), oA = __shfl_xor(A, 32);
        const float Mx = fmaxf(M, oM);
        if (Mx != -INFINITY) {
            const float a = exp2f(M - Mx), b = exp2f(oM - Mx);
            L = a * L + b * oL;
            A = a * A + b * oA;
        }
        M = Mx;
    }
    constexpr int kWavesM = kMergeGroups / 2;
    __shared__ float s_m[kWavesM][kMergeCols], s_l[kWavesM][kMergeCols], s_a[kWavesM][kMergeCols];
    const int wv = tid / 64, cc = tid % kMergeCols;
    if ((tid & 63) < kMergeCols) {
        s_m[wv][cc] = M;
        s_l[wv][cc] = L;
        s_a[wv][cc] = A;
    }
    __syncthreads();
    if (wv == 0) {
        const int k0 = (tid / kMergeCols) * (kWavesM / 2);
        float Mt = -INFINITY;
        for (int k = k0; k < k0 + kWavesM / 2; ++k) Mt = fmaxf(Mt, s_m[k][cc]);
        float Lt = 0.f, At = 0.f;
        if (Mt != -INFINITY) {
            for (int k = k0; k < k0 + kWavesM / 2; ++k) {
                const float a = exp2f(s_m[k][cc] - Mt);
                Lt += a * s_l[k][cc];
                At += a * s_a[k][cc];
            }
        }
        const float oM = __shfl_xor(Mt, 32), oL = __shfl_xor(Lt, 32), oA = __shfl_xor(At, 32);
        const float Mx = fmaxf(Mt, oM);
        if (Mx != -INFINITY) {
            const float a = exp2f(Mt - Mx), b = exp2f(oM - Mx);
            Lt = a * Lt + b * oL;
            At = a * At + b * oA;
        }
        if (tid < kMergeCols) out[row * kHeadDim + c] = Lt > 0.f ? At / Lt : 0.f;
    }
}

// Merge with the fp16 recent window (the recent tokens kept unquantized): per row
// (sequence, query head) and 32 output columns, the packed part's split partials are
// merged as above, then exact attention over the window tokens -- positions
// [len - nw, len), nw = min(len, window), each at ring row (position mod window), the
// newest from k_new/v_new when given -- is folded in as one more partial.  Logits are
// fp32 dot products of the binary16 values, in log2 units like the partials.  With
// k_new, one workgroup per (sequence, KV head) then writes the new token to its ring
// row; no workgroup of this launch reads that row (it held the token that left).
constexpr int kWindowMax = 1024;

__global__ __launch_bounds__(kMergeCols * kMergeGroups) void merge_window_kernel(const float* __restrict__ ws,
                                                                                  int n_split, float* __restrict__ out,
                                                                                  WindowArgs w) {
    const int64_t row = blockIdx.x;
    const int s = (int)(row / w.n_q), h = (int)(row % w.n_q), kvh = h / w.g;
    const int tid = threadIdx.x, sg = tid / kMergeCols, cc = tid % kMergeCols, c = blockIdx.y * kMergeCols + cc;
    constexpr int D2 = kHeadDim + 2;
    __shared__ float s_q[kHeadDim];
    __shared__ float s_z[kWindowMax];
    __shared__ float s_red[kMergeGroups][kMergeCols];
    __shared__ float s_m[kMergeGroups / 2][kMergeCols], s_l[kMergeGroups / 2][kMergeCols],
        s_a[kMergeGroups / 2][kMergeCols];
    __shared__ float s_wm, s_wl;
    const int64_t len = max((int64_t)w.seq_len[s], (int64_t)0);
    const int nw = (int)min(len, (int64_t)w.window);
    const int64_t t0 = len - nw;
    if (tid < kHeadDim) s_q[tid] = h2f(w.q[row * kHeadDim + tid]);
    auto krow = [&](int i) -> const uint16_t* {  // window token i (position t0 + i)
        const int64_t t = t0 + i;
        if (w.k_new && t == len - 1) return w.k_new + (int64_t)s * w.new_stride_seq + (int64_t)kvh * w.new_stride_head;
        return w.win_k + (((int64_t)s * w.n_kv + kvh) * w.window + t % w.window) * kHeadDim;
    };
    auto vrow = [&](int i) -> const uint16_t* {
        const int64_t t = t0 + i;
        if (w.v_new && t == len - 1) return w.v_new + (int64_t)s * w.new_stride_seq + (int64_t)kvh * w.new_stride_head;
        return w.win_v + (((int64_t)s * w.n_kv + kvh) * w.window + t % w.window) * kHeadDim;
    };

    // the window's K pieces (first 128 tokens: eight lanes per token) and V values
    // (four tokens per split group) go out with the partials' loads
    const int kj = tid & 7;
    uint4 kpre[2] = {uint4{0, 0, 0, 0}, uint4{0, 0, 0, 0}};
    if (tid / 8 < nw) {
        const uint4* kr = (const uint4*)krow(tid / 8) + 2 * kj;
        kpre[0] = kr[0];
        kpre[1] = kr[1];
    }
    constexpr int kVPre = 4;
    uint32_t vpre[kVPre];
#pragma unroll
    for (int u = 0; u < kVPre; ++u) vpre[u] = sg + kMergeGroups * u < nw ? vrow(sg + kMergeGroups * u)[c] : 0u;

    // ---- the packed part's partials (as merge_kernel)
    const float* part = ws + row * n_split * D2;
    float M = -INFINITY, L = 0.f, A = 0.f;
    for (int sp0 = sg; sp0 < n_split; sp0 += kMergeGroups * kMergeUnroll) {
        float m[kMergeUnroll], l[kMergeUnroll], o[kMergeUnroll];
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const int sp = sp0 + u * kMergeGroups;
            const float* p = part + (int64_t)min(sp, n_split - 1) * D2;
            m[u] = sp < n_split ? p[0] : -INFINITY;
            l[u] = p[1];
            o[u] = p[2 + c];
        }
        float mx = M;
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) mx = fmaxf(mx, m[u]);
        if (mx == -INFINITY) continue;
        const float r = exp2f(M - mx);
        L *= r;
        A *= r;
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const float a = exp2f(m[u] - mx);
            L += a * l[u];
            A += a * o[u];
        }
        M = mx;
    }
    {
        const float oM = __shfl_xor(M, 32), oL = __shfl_xor(L, 32), oA = __shfl_xor(A, 32);
        const float Mx = fmaxf(M, oM);
        if (Mx != -INFINITY) {
            const float a = exp2f(M - Mx), b = exp2f(oM - Mx);
            L = a * L + b * oL;
            A = a * A + b * oA;
        }
        M = Mx;
    }
    const int wv = tid / 64;
    if ((tid & 63) < kMergeCols) { s_m[wv][cc] = M; s_l[wv][cc] = L; s_a[wv][cc] = A; }
    __syncthreads();  // s_q ready too

    // ---- window logits: eight lanes per token, 16 coordinates each
    for (int i = tid / 8; i < nw; i += kMergeCols * kMergeGroups / 8) {
        const int j = kj;
        const uint4* kr = (const uint4*)krow(i) + 2 * j;
        float z = 0.f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint4 v4 = i == tid / 8 ? kpre[k] : kr[k];
            const uint32_t wd[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                z += s_q[16 * j + 8 * k + 2 * e] * h2f(wd[e] & 0xffffu);
                z += s_q[16 * j + 8 * k + 2 * e + 1] * h2f(wd[e] >> 16);
            }
        }
        z += __shfl_xor(z, 1);
        z += __shfl_xor(z, 2);
        z += __shfl_xor(z, 4);
        if (j == 0) s_z[i] = z * w.scale_log2;
    }
    __syncthreads();
    {  // window max, then weight sum: per wave, then across the 16 waves
        float mx = tid < nw ? s_z[tid] : -INFINITY;
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        if ((tid & 63) == 0) s_red[0][wv] = mx;
        __syncthreads();
        mx = s_red[0][tid & 15];
        for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
        float l = (tid < nw && mx != -INFINITY) ? exp2f(s_z[tid] - mx) : 0.f;
        if (tid < nw) s_z[tid] = l;  // the weights themselves from here on
        for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
        if ((tid & 63) == 0) s_red[1][wv] = l;
        __syncthreads();
        if (tid == 0) {
            float t = 0.f;
            for (int k = 0; k < kMergeGroups / 2; ++k) t += s_red[1][k];
            s_wm = mx;
            s_wl = t;
        }
    }
    __syncthreads();
    const float wm = s_wm, wl = s_wl;
    // window output for column c: group sg takes tokens sg, sg + 32, ...
    float oacc = 0.f;
#pragma unroll
    for (int u = 0; u < kVPre; ++u)
        if (sg + kMergeGroups * u < nw) oacc += s_z[sg + kMergeGroups * u] * h2f(vpre[u]);
    for (int i = sg + kMergeGroups * kVPre; i < nw; i += kMergeGroups) oacc += s_z[i] * h2f(vrow(i)[c]);
    __syncthreads();  // s_red's rows 0 and 1 were read above
    s_red[sg][cc] = oacc;
    __syncthreads();
    if (wv == 0) {
        const int k0 = (tid / kMergeCols) * (kMergeGroups / 4);
        float Mt = -INFINITY;
        for (int k = k0; k < k0 + kMergeGroups / 4; ++k) Mt = fmaxf(Mt, s_m[k][cc]);
        float Lt = 0.f, At = 0.f;
        if (Mt != -INFINITY) {
            for (int k = k0; k < k0 + kMergeGroups / 4; ++k) {
                const float a = exp2f(s_m[k][cc] - Mt);
                Lt += a * s_l[k][cc];
                At += a * s_a[k][cc];
            }
        }
        const float oM = __shfl_xor(Mt, 32), oL = __shfl_xor(Lt, 32), oA = __shfl_xor(At, 32);
        float Mx = fmaxf(Mt, oM);
        if (Mx != -INFINITY) {
            const float a = exp2f(Mt - Mx), b = exp2f(oM - Mx);
            Lt = a * Lt + b * oL;
            At = a * At + b * oA;
        }
        if (tid < kMergeCols) {
            float ow = 0.f;
            for (int k = 0; k < kMergeGroups; ++k) ow += s_red[k][cc];
            const float M2 = fmaxf(Mx, wm);
            if (M2 != -INFINITY) {
                const float a = exp2f(Mx - M2), b = exp2f(wm - M2);
                Lt = a * Lt + b * wl;
                At = a * At + b * ow;
            }
            out[row * kHeadDim + c] = Lt > 0.f ? At / Lt : 0.f;
        }
    }
    // ---- the new token into its ring row (one workgroup per sequence and KV head)
    if (w.k_new && len > 0 && h % w.g == 0 && blockIdx.y == 0 && tid < 2 * (kHeadDim / 2)) {
        const bool isv = tid >= kHeadDim / 2;
        const int e = tid & (kHeadDim / 2 - 1);
        const uint16_t* src = (isv ? w.v_new : w.k_new) + (int64_t)s * w.new_stride_seq + (int64_t)kvh * w.new_stride_head;
        uint16_t* dst = (isv ? w.win_v : w.win_k) + (((int64_t)s * w.n_kv + kvh) * w.window + (len - 1) % w.window) * kHeadDim;
        ((uint32_t*)dst)[e] = ((const uint32_t*)src)[e];
    }
}

hipError_t launch_decode_mfma(const kvq_geom& g, const DecodePlan& plan, int n_q_heads, const uint16_t* q,
                              uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len, int n_seq,
                              int64_t max_len, const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                              float scale_log2, float* workspace, hipStream_t st, const AppendArgs& app);

int mfma_blocks_per_cu(const kvq_geom& g);

// compute units of the current device (256 if it cannot be queried)
static int device_cus() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

int plan_decode(const kvq_geom& g, int n_q_heads, int n_seq, int64_t max_len, int kernel, int tiles_per_split,
                DecodePlan* plan) {
    const int grp = n_q_heads / g.n_kv_heads;
    // the matrix-core kernel keeps a K record (<= 64 bytes: k_budget <= 256) in registers
    const bool mfma_ok = kMfmaKernel && g.k_budget <= 4 * kMaxBlocks && g.v_bits <= 8 && grp <= 8;
    if (kernel == KVQ_DECODE_AUTO) kernel = mfma_ok ? KVQ_DECODE_MFMA : KVQ_DECODE_GENERIC;
    if (kernel == KVQ_DECODE_MFMA && !mfma_ok) return KVQ_ERR_SHAPE;
    if (kernel == KVQ_DECODE_GENERIC && grp > kGenericMaxGroup) return KVQ_ERR_SHAPE;
    if (kernel != KVQ_DECODE_MFMA && kernel != KVQ_DECODE_GENERIC) return KVQ_ERR_ARG;
    const int64_t n_tiles = (max_len + kTile - 1) / kTile;
    int64_t T = tiles_per_split;
    if (T <= 0 && kernel == KVQ_DECODE_MFMA) {
        // One pass of resident workgroups: every wave of the grid gets the same
        // whole number of tiles (chunks are a multiple of the 4 waves), as few as
        // the chip's resident waves allow.
        const int64_t units = (int64_t)n_seq * g.n_kv_heads;
        const int64_t slots = (int64_t)device_cus() * std::max(1, mfma_blocks_per_cu(g));
        int64_t per_wave = std::max<int64_t>(1, (units * n_tiles + 4 * slots - 1) / (4 * slots));
        while (units * ((n_tiles + 4 * per_wave - 1) / (4 * per_wave)) > slots && 4 * per_wave < n_tiles) ++per_wave;
        T = 4 * per_wave;
    } else if (T <= 0) {
        // enough chunks to give every CU several workgroups
        const int64_t units = (int64_t)n_seq * g.n_kv_heads;
        const int64_t target = 512;
        int64_t want = (target + units - 1) / (units > 0 ? units : 1);
        if (want < 1) want = 1;
        T = std::max<int64_t>(1, (n_tiles + want - 1) / want);
    }
    int64_t ns = n_tiles > 0 ? (n_tiles + T - 1) / T : 1;
    if (ns > 65535) return KVQ_ERR_CAPACITY;
    plan->kernel = kernel;
    plan->tiles_per_split = (int)T;
    plan->n_split = (int)ns;
    plan->workspace = (int64_t)n_seq * n_q_heads * ns * (kHeadDim + 2) * 4;
    return 0;
}

hipError_t launch_decode_partials(const kvq_geom& g, const DecodePlan& plan, int n_q_heads, const uint16_t* q,
                                  uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len,
                                  int n_seq, int64_t max_len, const uint8_t* k_bits, const float* k_sigma,
                                  const float* v_sigma, float softmax_scale, float* partials, hipStream_t st,
                                  const AppendArgs& app) {
    const float scale_log2 = softmax_scale * kLog2e;
    const int grp = n_q_heads / g.n_kv_heads;
    // the matrix-core kernel appends inside (the tail tile's wave); the generic one
    // gets the append as a kernel of its own first
    if (plan.kernel == KVQ_DECODE_MFMA)
        return launch_decode_mfma(g, plan, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, max_len, k_bits,
                                  k_sigma, v_sigma, scale_log2, partials, st, app);
    if (app.k) {
        const hipError_t e = launch_append_step(g, n_seq, app, seq_len, k_bits, k_sigma, v_sigma, cache,
                                                seq_byte_off, st);
        if (e != hipSuccess) return e;
    }
    dim3 grid(plan.n_split, g.n_kv_heads, n_seq);
    hipLaunchKernelGGL(decode_generic_kernel, grid, dim3(256), 0, st, q, cache, seq_byte_off, seq_len, max_len,
                       g.capacity_tokens, k_bits, k_sigma, v_sigma, scale_log2, n_q_heads, grp, g.rope_pairing,
                       g.k_budget, g.v_bits, plan.tiles_per_split, plan.n_split, partials, app.window);
    return hipGetLastError();
}

hipError_t launch_merge_window(int n_seq, int n_split, const float* partials, float* out, const WindowArgs& w,
                               hipStream_t st) {
    hipLaunchKernelGGL(merge_window_kernel, dim3(n_seq * w.n_q, kHeadDim / kMergeCols), dim3(kMergeCols * kMergeGroups),
                       0, st, partials, n_split, out, w);
    return hipGetLastError();
}

hipError_t launch_merge(int n_rows, int n_split, const float* partials, float* out, hipStream_t st) {
    hipLaunchKernelGGL(merge_kernel, dim3(n_rows, kHeadDim / kMergeCols), dim3(kMergeCols * kMergeGroups), 0, st,
                       partials, n_split, out);
    return hipGetLastError();
}

}  // namespace kvq
