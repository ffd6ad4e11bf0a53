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
    int pairing, int k_budget, int v_bits, int tiles_per_split, int n_split, float* __restrict__ ws,
    AppendArgs app) {
    const int split = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x;
    __shared__ float s_x[kTile][kHeadDim + 1];  // dequantized K, then V, of the current tile
    if (app.window > 0 && split >= n_split - window_chunks(app.window)) {  // the fp16 window's chunks
        window_chunk<kGenericMaxGroup>(app, q, n_q, g, s, kvh, seq_len, scale_log2, ws, n_split,
                                       split - (n_split - window_chunks(app.window)), &s_x[0][0]);
        return;
    }
    // packed tokens (seq_len less the fp16 window, if any)
    const int64_t len = min(max((int64_t)seq_len[s] - app.window, (int64_t)0), max_len);
    const int64_t n_tiles_seq = (len + kTile - 1) / kTile;
    const int64_t t0 = (int64_t)split * tiles_per_split;
    const int64_t t1 = min(t0 + tiles_per_split, n_tiles_seq);
    const int D2 = kHeadDim + 2;

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

// grid: (n_seq * n_q rows, 16 groups of 8 coordinates); block: 256 threads = 32 split groups x 8 coordinates
// Split merge: out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j.  A workgroup
// takes 8 coordinates of one row, so a row's merge spreads over 16 compute units;
// its 32 split groups stride over the splits with their own running maximum,
// sixteen splits' loads in flight at a time (512 splits in one pass).  A wave's
// eight split groups (lanes 8 apart) combine by lane swaps, the four waves through LDS.
constexpr int kMergeCols = 8, kMergeGroups = 32, kMergeUnroll = 16;

__device__ __forceinline__ void merge_pair(float& M, float& L, float& A, float oM, float oL, float oA) {
    const float Mx = fmaxf(M, oM);
    if (Mx != -INFINITY) {
        const float a = exp2f(M - Mx), b = exp2f(oM - Mx);
        L = a * L + b * oL;
        A = a * A + b * oA;
    }
    M = Mx;
}

__global__ __launch_bounds__(kMergeCols * kMergeGroups) void merge_kernel(const float* __restrict__ ws, int n_split,
                                                                           float* __restrict__ out) {
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, sg = tid / kMergeCols, cc = tid % kMergeCols, c = blockIdx.y * kMergeCols + cc;
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
    // the wave's eight split groups: lanes l, l ^ 8, l ^ 16, l ^ 32 ... share a coordinate
#pragma unroll
    for (int mask = kMergeCols; mask < 64; mask <<= 1)
        merge_pair(M, L, A, __shfl_xor(M, mask), __shfl_xor(L, mask), __shfl_xor(A, mask));
    constexpr int kWavesM = kMergeCols * kMergeGroups / 64;
    __shared__ float s_m[kWavesM][kMergeCols], s_l[kWavesM][kMergeCols], s_a[kWavesM][kMergeCols];
    const int wv = tid / 64;
    if ((tid & 63) < kMergeCols) {
        s_m[wv][cc] = M;
        s_l[wv][cc] = L;
        s_a[wv][cc] = A;
    }
    __syncthreads();
    if (tid < kMergeCols) {
        float Mt = s_m[0][cc], Lt = s_l[0][cc], At = s_a[0][cc];
#pragma unroll
        for (int k = 1; k < kWavesM; ++k) merge_pair(Mt, Lt, At, s_m[k][cc], s_l[k][cc], s_a[k][cc]);
        out[row * kHeadDim + c] = Lt > 0.f ? At / Lt : 0.f;
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
    const int n_chunks = plan.n_split + (app.window > 0 ? window_chunks(app.window) : 0);  // + the window's
    dim3 grid(n_chunks, g.n_kv_heads, n_seq);
    hipLaunchKernelGGL(decode_generic_kernel, grid, dim3(256), 0, st, q, cache, seq_byte_off, seq_len, max_len,
                       g.capacity_tokens, k_bits, k_sigma, v_sigma, scale_log2, n_q_heads, grp, g.rope_pairing,
                       g.k_budget, g.v_bits, plan.tiles_per_split, n_chunks, partials, app);
    return hipGetLastError();
}

// The same merge for a few splits per row (the prefill's key-range splits): thread
// (row, coordinate), two rows per workgroup, every split's partial in one pass with
// a running maximum.
constexpr int kMergeSmallMax = 16;
__global__ __launch_bounds__(2 * kHeadDim) void merge_small_kernel(const float* __restrict__ ws, int n_split,
                                                                   int64_t n_rows, float* __restrict__ out) {
    const int64_t row = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
    const int c = threadIdx.x & (kHeadDim - 1);
    if (row >= n_rows) return;
    constexpr int D2 = kHeadDim + 2;
    const float* part = ws + row * n_split * D2;
    float m[kMergeSmallMax], l[kMergeSmallMax], o[kMergeSmallMax];
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMergeSmallMax; ++j) {
        if (j < n_split) {
            m[j] = part[j * D2];
            l[j] = part[j * D2 + 1];
            o[j] = part[j * D2 + 2 + c];
            M = fmaxf(M, m[j]);
        }
    }
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int j = 0; j < kMergeSmallMax; ++j) {
            if (j < n_split) {
                const float a = exp2f(m[j] - M);
                L += a * l[j];
                A += a * o[j];
            }
        }
    }
    out[row * kHeadDim + c] = L > 0.f ? A / L : 0.f;
}

hipError_t launch_merge(int n_rows, int n_split, const float* partials, float* out, hipStream_t st) {
    if (n_split <= kMergeSmallMax) {
        hipLaunchKernelGGL(merge_small_kernel, dim3((n_rows + 1) / 2), dim3(2 * kHeadDim), 0, st, partials, n_split,
                           (int64_t)n_rows, out);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(merge_kernel, dim3(n_rows, kHeadDim / kMergeCols), dim3(kMergeCols * kMergeGroups), 0, st,
                       partials, n_split, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------- read-bandwidth probe
// A plain streaming read of n16 16-byte words: every thread keeps eight 128-bit loads
// in flight over a grid-stride loop and folds them with XOR; one word per workgroup
// is written so the loads stay live.  It measures the read rate a simple kernel
// reaches on this device (the ceiling the attention kernels are compared with).
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[i + u * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t s_acc[256];
    s_acc[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int t = 0; t < 256; ++t) r ^= s_acc[t];
        sink[blockIdx.x] = r;
    }
}

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, int n_blocks, hipStream_t st) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(n_blocks), dim3(256), 0, st, (const uint4*)src, bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace kvq
