// kvq_energy_alloc.hip -- block energy (exact 128-bit integer reduction) and
// greedy bit allocation, for "RoPE-Aware Bit Allocation for KV-Cache
// Quantization" (abstract: per layer and KV head, a label-free energy score per
// RoPE block, then integer widths handed out greedily by marginal gain).
#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {

// ---------------------------------------------------------------------------
// Block energy
// ---------------------------------------------------------------------------
// A binary16 pattern with exponent field e and fraction m is M * 2^(e-25) with
// M = 1024 + m (e >= 1), or m * 2^-24 (e = 0).  Its square is M^2 << sh(e) units of
// 2^-48, sh(e) = max(2e - 2, 0): an integer below 2^82.  A workgroup sums M^2 per
// (coordinate, exponent) in 32-bit LDS counters (M^2 < 2^22 and at most 1024 rows
// per workgroup keep every counter below 2^32), then forms each coordinate's
// 128-bit total as the sum of counter << sh(e) -- exact, and a handful of
// instructions per element instead of a 128-bit add.

// 128-bit add of (alo, ahi) into a (lo, hi) pair in global memory with two 64-bit
// atomics: the carry out of the low word is forwarded to the high word, so the
// final value is exact whatever the interleaving.
__device__ __forceinline__ void atomic_add_u128(uint64_t* p, uint64_t alo, uint64_t ahi) {
    const uint64_t old = atomicAdd((unsigned long long*)p, (unsigned long long)alo);
    const uint64_t carry = (old + alo < old) ? 1ull : 0ull;
    if (ahi + carry) atomicAdd((unsigned long long*)(p + 1), (unsigned long long)(ahi + carry));
}

constexpr int kEnergyMaxRows = 1024;  // rows per workgroup (keeps the 32-bit counters exact)
constexpr int kHistStride = 33;       // counters per coordinate: 32 exponents + 1 (bank spread)

__device__ __forceinline__ void hist_add(uint32_t* hist_c, uint32_t h) {
    const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
    const uint32_t M = e ? (1024u | m) : m;
    atomicAdd(hist_c + e, M * M);
}

// grid: (n_heads, row blocks); block: 1024 threads = 16 row lanes x 64 coordinate
// pairs.  Thread (r, j) reads coordinates 2j, 2j+1 of rows r, r+16, ... of its row
// range, sixteen rows per batch.  Few, large workgroups: every workgroup ends in one
// 128-bit atomic per block, and those atomics all meet in the head's 64 counters.
constexpr int kEnergyRowLanes = 16;
constexpr int kEnergyThreads = 64 * kEnergyRowLanes;

__global__ __launch_bounds__(kEnergyThreads) void block_energy_kernel(const uint16_t* __restrict__ x, int64_t n_tok,
                                                          int64_t stride_tok, int64_t stride_head, int d,
                                                          int pairing, int64_t rows_per_block,
                                                          uint64_t* __restrict__ energy) {
    __shared__ uint32_t s_hist[kHeadDim * kHistStride];
    __shared__ uint64_t s_lo[kHeadDim], s_hi[kHeadDim];
    const int h = blockIdx.x;
    const int j = threadIdx.x & 63;
    const int r = threadIdx.x >> 6;  // row lane
    const int npairs = d >> 1;
    for (int i = threadIdx.x; i < kHeadDim * kHistStride; i += kEnergyThreads) s_hist[i] = 0u;
    __syncthreads();
    const int64_t row0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t row1 = min(row0 + rows_per_block, n_tok);
    if (j < npairs) {
        const uint16_t* base = x + (int64_t)h * stride_head + 2 * j;
        uint32_t* h0 = s_hist + (2 * j) * kHistStride;
        uint32_t* h1 = h0 + kHistStride;
        int64_t t = row0 + r;
        constexpr int RL = kEnergyRowLanes;
        for (; t + 15 * RL < row1; t += 16 * RL) {
            uint32_t w[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) w[k] = *(const uint32_t*)(base + (t + RL * k) * stride_tok);
#pragma unroll
            for (int k = 0; k < 16; ++k) { hist_add(h0, w[k] & 0xffffu); hist_add(h1, w[k] >> 16); }
        }
        for (; t + 3 * RL < row1; t += 4 * RL) {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = *(const uint32_t*)(base + (t + RL * k) * stride_tok);
#pragma unroll
            for (int k = 0; k < 4; ++k) { hist_add(h0, w[k] & 0xffffu); hist_add(h1, w[k] >> 16); }
        }
        for (; t < row1; t += RL) {
            const uint32_t w0 = *(const uint32_t*)(base + t * stride_tok);
            hist_add(h0, w0 & 0xffffu); hist_add(h1, w0 >> 16);
        }
    }
    __syncthreads();
    // coordinate totals: sum over exponents of counter << sh(e)
    if ((int)threadIdx.x < 2 * npairs) {
        const uint32_t* hc = s_hist + threadIdx.x * kHistStride;
        uint64_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
            const uint64_t v = hc[e];
            const int sh = e ? 2 * e - 2 : 0;
            const uint64_t l = v << sh;
            const uint64_t u = sh > 32 ? v >> (64 - sh) : 0ull;
            lo += l;
            hi += u + (lo < l ? 1ull : 0ull);
        }
        s_lo[threadIdx.x] = lo;
        s_hi[threadIdx.x] = hi;
    }
    __syncthreads();
    if ((int)threadIdx.x < npairs) {
        const int i = threadIdx.x;
        const int p = pairing == KVQ_PAIR_HALF ? i : 2 * i;
        const int q = pairing == KVQ_PAIR_HALF ? i + npairs : 2 * i + 1;
        uint64_t lo = s_lo[p], hi = s_hi[p];
        lo += s_lo[q];
        hi += s_hi[q] + (lo < s_lo[q] ? 1ull : 0ull);
        if (lo | hi) atomic_add_u128(energy + ((int64_t)h * npairs + i) * 2, lo, hi);
    }
}

hipError_t launch_block_energy(const uint16_t* x, int64_t n_tok, int64_t stride_tok, int64_t stride_head,
                               int n_heads, int d, int pairing, uint64_t* energy, hipStream_t st) {
    // about 512 workgroups in total, 256 .. kEnergyMaxRows rows each
    const int64_t blocks_per_head = (512 + n_heads - 1) / n_heads;
    int64_t rows = (n_tok + blocks_per_head - 1) / blocks_per_head;
    if (rows < 256) rows = 256;
    rows = (rows + 15) / 16 * 16;
    if (rows > kEnergyMaxRows) rows = kEnergyMaxRows;
    const int64_t nby = (n_tok + rows - 1) / rows;
    dim3 grid(n_heads, (unsigned)nby);
    hipLaunchKernelGGL(block_energy_kernel, grid, dim3(kEnergyThreads), 0, st, x, n_tok, stride_tok, stride_head, d, pairing,
                       rows, energy);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation
// ---------------------------------------------------------------------------
// unsigned 128-bit integer -> double, round to nearest even
__device__ __forceinline__ double u128_to_f64(uint64_t lo, uint64_t hi) {
    if (hi == 0 && lo < (1ull << 53)) return (double)lo;  // exact
    const int top = hi ? 127 - __clzll(hi) : 63 - __clzll(lo);
    const int drop = top - 52;  // 1..75 bits below the kept 53
    uint64_t keep;
    if (drop >= 64) keep = hi >> (drop - 64);
    else keep = (hi << (64 - drop)) | (lo >> drop);
    const int rb = drop - 1;  // round bit position
    const uint64_t round_bit = rb >= 64 ? (hi >> (rb - 64)) & 1ull : (lo >> rb) & 1ull;
    bool sticky;
    if (rb >= 64) sticky = lo != 0 || (rb > 64 && (hi & ((1ull << (rb - 64)) - 1ull)) != 0);
    else sticky = rb > 0 && (lo & ((1ull << rb) - 1ull)) != 0;
    if (round_bit && (sticky || (keep & 1ull))) keep += 1;
    return ldexp((double)keep, drop);
}

// Workgroups (unit, part): wave 0 (lane i = block i) of every part forms E_i and E_tot,
// part 0 writes sigma (and the widths of the uniform mode).  Greedy: step after step
// the block with the largest marginal gain E_i * dD[b_i] (lowest index on ties) gains
// one bit.  A block's gains fall strictly with its width (dD strictly decreasing; all
// zero when E_i = 0), so the candidate (i, w) is always taken after (i, w - 1), and
// the greedy order is the order of all 8 nb candidates (i, w) by gain descending, then
// block, then width ascending: the first `budget` of them are taken, and b_i counts
// block i's.  Part p ranks the candidates of blocks 8p .. 8p+7, wave w block 8p + w:
// eight threads per candidate each count the candidates that precede it among 64 of
// the 512 (rank = #{j : key_j > key, or key_j == key and j < own index}), and the
// eight counts are summed across the lanes.
constexpr int kAllocThreads = 8 * 64;
constexpr int kAllocBlocksPerPart = kAllocThreads / 64;

__global__ __launch_bounds__(kAllocThreads) void allocate_kernel(const uint64_t* __restrict__ energy, int nb,
                                                                int budget, int mode, uint8_t* __restrict__ bits,
                                                                float* __restrict__ sigma) {
    __shared__ double s_E[64];
    __shared__ uint64_t s_key[kAllocThreads];
    const int u = blockIdx.x, part = blockIdx.y, tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (wave == 0) {
        const int i = tid;
        const bool act = i < nb;
        const uint64_t lo = act ? energy[((int64_t)u * nb + i) * 2] : 0ull;
        const uint64_t hi = act ? energy[((int64_t)u * nb + i) * 2 + 1] : 0ull;
        const double E = ldexp(u128_to_f64(lo, hi), -48);
        s_E[i] = E;
        if (part == 0) {
            uint64_t tlo = lo, thi = hi;
            for (int off = 32; off >= 1; off >>= 1) {
                const uint64_t olo = __shfl_xor(tlo, off), ohi = __shfl_xor(thi, off);
                tlo += olo;
                thi += ohi + (tlo < olo ? 1ull : 0ull);
            }
            const double Etot = ldexp(u128_to_f64(tlo, thi), -48);
            if (act) {
                sigma[(int64_t)u * nb + i] = Etot > 0.0 ? (float)sqrt(E / (2.0 * Etot)) : 0.0f;
                if (budget == 16 * nb) bits[(int64_t)u * nb + i] = 16;
                else if (mode == KVQ_UNIFORM) bits[(int64_t)u * nb + i] = (uint8_t)(budget / nb);
            }
        }
    }
    if (budget == 16 * nb || mode == KVQ_UNIFORM) return;  // uniform over the workgroup
    __syncthreads();
    {
        // gains are >= 0, so their bit patterns order like the values; candidates of
        // absent blocks get gain 0 and the largest indices, so they precede nobody
        const int i = tid >> 3, w = tid & 7;
        const double gain = i < nb ? s_E[i] * (double)c_gain_dd[w] : 0.0;
        s_key[tid] = __double_as_longlong(gain);
    }
    __syncthreads();
    const int cand = 64 * part + (tid >> 3), sub = tid & 7;
    const uint64_t key = s_key[cand];
    int rank = 0;
    for (int j = 64 * sub; j < 64 * sub + 64; j += 2) {
        const uint64_t a = s_key[j], b2 = s_key[j + 1];
        rank += (a > key || (a == key && j < cand)) ? 1 : 0;
        rank += (b2 > key || (b2 == key && j + 1 < cand)) ? 1 : 0;
    }
    rank += __shfl_xor(rank, 1);
    rank += __shfl_xor(rank, 2);
    rank += __shfl_xor(rank, 4);
    const unsigned long long taken = __ballot(sub == 0 && rank < budget);
    const int blk = kAllocBlocksPerPart * part + wave;
    if ((tid & 63) == 0 && blk < nb) bits[(int64_t)u * nb + blk] = (uint8_t)__popcll(taken);
}

hipError_t launch_allocate(const uint64_t* energy, int n_units, int nb, int budget, int mode, uint8_t* bits,
                           float* sigma, hipStream_t st) {
    const bool greedy = !(budget == 16 * nb || mode == KVQ_UNIFORM);
    const int parts = greedy ? (nb + kAllocBlocksPerPart - 1) / kAllocBlocksPerPart : 1;
    hipLaunchKernelGGL(allocate_kernel, dim3(n_units, parts), dim3(kAllocThreads), 0, st, energy, nb, budget, mode,
                       bits, sigma);
    return hipGetLastError();
}

}  // namespace kvq
