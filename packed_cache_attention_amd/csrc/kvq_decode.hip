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

// grid: (n_seq * n_q rows, 16 groups of 8 coordinates); block: 256 threads = 32 split groups x 8 coordinates
// Split merge: out = sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j.  A workgroup
// takes 8 coordinates of one row, so a row's merge spreads over 16 compute units;
// its 32 split groups stride over the splits with their own running maximum,
// sixteen splits' loads in flight at a time (512 splits in one pass).  A wave's
// eight split groups (lanes 8 apart) combine by DPP and permlane exchanges, the four
// waves through LDS.  Weights 2^(m_j - M) use the hardware exp2 (arguments <= 0; a
// weight below 2^-126 is negligible beside the largest, which is 1).
constexpr int kMergeCols = 8, kMergeGroups = 32, kMergeUnroll = 16;

__device__ __forceinline__ void merge_pair(float& M, float& L, float& A, float oM, float oL, float oA) {
    const float Mx = fmaxf(M, oM);
    if (Mx != -INFINITY) {
        const float a = __builtin_amdgcn_exp2f(M - Mx), b = __builtin_amdgcn_exp2f(oM - Mx);
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
            const int off = min(sp, n_split - 1) * D2;  // within the row's partials (32-bit)
            m[u] = sp < n_split ? part[off] : -INFINITY;
            l[u] = part[off + 1];
            o[u] = part[off + 2 + c];
        }
        float mx = M;
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) mx = fmaxf(mx, m[u]);
        if (mx == -INFINITY) continue;  // nothing attended yet in these splits
        const float r = __builtin_amdgcn_exp2f(M - mx);
        L *= r;
        A *= r;
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const float a = __builtin_amdgcn_exp2f(m[u] - mx);
            L += a * l[u];
            A += a * o[u];
        }
        M = mx;
    }
    // the wave's eight split groups: lanes l, l ^ 8, l ^ 16, l ^ 32 share a coordinate;
    // each exchange hands both lanes the same two operands in the same order (the
    // lower lane's first), so both hold the same merged triple
    {
        const float pM = dpp_ror8(M), pL = dpp_ror8(L), pA = dpp_ror8(A);
        const bool up = (tid & 8) != 0;
        float M0 = up ? pM : M, L0 = up ? pL : L, A0 = up ? pA : A;
        merge_pair(M0, L0, A0, up ? M : pM, up ? L : pL, up ? A : pA);
        M = M0; L = L0; A = A0;
    }
    {
        float m0, m1, l0, l1, a0, a1;
        pair16(M, m0, m1); pair16(L, l0, l1); pair16(A, a0, a1);
        merge_pair(m0, l0, a0, m1, l1, a1);
        M = m0; L = l0; A = a0;
    }
    {
        float m0, m1, l0, l1, a0, a1;
        pair32(M, m0, m1); pair32(L, l0, l1); pair32(A, a0, a1);
        merge_pair(m0, l0, a0, m1, l1, a1);
        M = m0; L = l0; A = a0;
    }
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
    const bool mfma_ok = kMfmaKernel && g.k_budget <= 4 * kMaxBlocks && (g.v_bits <= 8 || g.v_bits == 16) && grp <= 8;
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
        // the same one-pass rule for the generic kernel (one wave per tile, four per chunk)
        const int64_t units = (int64_t)n_seq * g.n_kv_heads;
        const int64_t slots = (int64_t)device_cus() * std::max(1, generic_blocks_per_cu(g, n_q_heads));
        int64_t per_wave = std::max<int64_t>(1, (units * n_tiles + 4 * slots - 1) / (4 * slots));
        while (units * ((n_tiles + 4 * per_wave - 1) / (4 * per_wave)) > slots && 4 * per_wave < n_tiles) ++per_wave;
        T = 4 * per_wave;
    }
    int64_t ns = n_tiles > 0 ? (n_tiles + T - 1) / T : 1;
    if (ns > 65535) return KVQ_ERR_CAPACITY;
    plan->kernel = kernel;
    plan->tiles_per_split = (int)T;
    plan->n_split = (int)ns;
    plan->table_bytes = kernel == KVQ_DECODE_GENERIC ? generic_table_bytes(g, n_q_heads, n_seq) : 0;
    plan->workspace = (int64_t)n_seq * n_q_heads * ns * (kHeadDim + 2) * 4 + plan->table_bytes;
    return 0;
}

hipError_t launch_decode_partials(const kvq_geom& g, const DecodePlan& plan, int n_q_heads, const uint16_t* q,
                                  uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len,
                                  int n_seq, int64_t max_len, const uint8_t* k_bits, const float* k_sigma,
                                  const float* v_sigma, float softmax_scale, float* partials, hipStream_t st,
                                  const AppendArgs& app) {
    const float scale_log2 = softmax_scale * kLog2e;
    // the matrix-core kernel appends inside (the tail tile's wave); the generic one in
    // the launch that builds its query table (one wave per (sequence, KV head))
    if (plan.kernel == KVQ_DECODE_MFMA)
        return launch_decode_mfma(g, plan, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, max_len, k_bits,
                                  k_sigma, v_sigma, scale_log2, partials, st, app);
    const int n_chunks = plan.n_split + (app.window > 0 ? window_chunks(app.window) : 0);  // + the window's
    return launch_decode_generic(g, plan.tiles_per_split, n_chunks, n_q_heads, q, cache, seq_byte_off, seq_len,
                                 n_seq, max_len, k_bits, k_sigma, v_sigma, scale_log2, partials, st, app);
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
