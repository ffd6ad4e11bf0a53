// kvq_prefill.hip -- chunked prefill attention over the packed cache (causal) on
// the CDNA4 matrix cores, for the packed-cache serving path of "RoPE-Aware Bit
// Allocation for KV-Cache Quantization" (abstract: at 256K and 512K only the packed
// cache fits; such a prompt is read here as filled chunk by chunk, each chunk's
// queries attending everything packed so far).
//
// A chunk of queries of one sequence sits at positions q_start .. q_start+n_q-1;
// query j attends slots [0, q_start + j] of the packed cache (the chunk is packed
// before the call), with the decode path's arithmetic: logits
//   z = s_t * sum_c (q_c sigma_c scale log2e) level[code_{t,c}]
// and o = sum_t 2^(z_t - m) s^V_t level[vcode_{t,c}], times sigma^V_c at the end.
//
// One workgroup = 256 query rows (8 waves x 32) of one (sequence, KV head): row r
// is query token r / g, head r % g of the group.  Per 64-slot tile the workgroup
// dequantizes K and V once into LDS as exact binary16 levels (K in K order, the
// query operand permuted to match), then every wave runs
//   S^T[key][row] = K . q'^T          v_mfma_f32_32x32x16_f16, q' split hi + lo
//   O^T[coord][row] += V^T . P'^T     v_mfma_f32_32x32x16_f16, P' = p.s^V split hi + lo
// (both operands split so that products keep about 22 bits, as in decode: a single
// binary16 weight would move the output by up to 2^-11 of the weighted values,
// which values cancelling across all coordinates could blow past the tolerance).
// The QK accumulator holds a column (query row) per lane, so its row max is a lane
// local max plus one permlane32 swap, and the accumulator itself, converted to
// binary16, is the B operand of PV (keys permuted to the accumulator's row order,
// the V operand read in the same order).  The running max is lazy (moves when a
// row's tile max exceeds it by more than 8 in log2 units), and the reference carries
// the decode kernel's power of two e (R = m + e, every s^V seen so far at most
// 2^(7+e)), so the binary16 operand p.s^V.2^-e stays below 2^15 for any binary16
// value rows (e = 0 for value norms below 2^7).  Tiles stream HBM -> LDS
// with global_load_lds_dwordx4, double-buffered.  Long key ranges split over
// workgroups into the decode path's partial format (merged by the same merge).
#include "kvq_decode_mfma.h"

namespace kvq {

constexpr int kPfWaves = 8;                  // waves per workgroup, 32 query rows each
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRows = 32 * kPfWaves;       // query rows per workgroup
constexpr int kPfKS = kHeadDim + 8;          // binary16 per dequantized K row (272 B: conflict-free b128 reads)
constexpr int kPfVS = kTile + 4;             // binary16 per dequantized V row (136 B: conflict-free b64 reads)
constexpr int kPfMaxTB = kTile * 256 + kHeadDim * 8 * 16 + 2 * kTile * 4;  // largest tile (K16, V16 passthrough)
constexpr int kPfChunks = kPfMaxTB / 16;
constexpr int kPfDmaPerThread = (kPfChunks + kPfThreads - 1) / kPfThreads;
constexpr float kPfSlack = 8.f;
constexpr int kPfMaxGroup = 128;             // query heads per KV head served
static_assert(kPfMaxGroup <= kPfRows, "a workgroup holds at least one query token");

struct PfSmem {
    // the workgroup's query rows (binary16 [rows][128]) are staged over stage, kd and vd
    // during the prologue
    alignas(16) uint8_t stage[2][kPfMaxTB];  // packed tiles, double-buffered
    alignas(16) uint16_t kd[kTile * kPfKS];   // dequantized K [key][K-order position]
    alignas(16) uint16_t vd[kHeadDim * kPfVS];// dequantized V [coordinate][key]
    uint32_t vpair[1024];    // value widths <= 5: entry a | b << v = levels (a, b) as a binary16 pair
    uint16_t lev[512];       // binary16 levels, width w at KVQ_CB_OFF(w)
    float fsig[kHeadDim];    // K-order position -> sigma^K of its block times scale log2e (0 past the fields)
    uint8_t fcoord[kHeadDim];// K-order position -> coordinate
    float vsig[kHeadDim];    // coordinate -> sigma^V
};
static_assert(2 * kPfMaxTB + sizeof(uint16_t) * (kTile * kPfKS + kHeadDim * kPfVS) >= kPfRows * kHeadDim * 2,
              "the query rows are staged over the tile buffers");
static_assert(kTile % kPfWaves == 0 && (kTile / kPfWaves) % 8 == 0 && (kHeadDim / kPfWaves) % 16 == 0,
              "dequantization shares: whole batches of eight keys / coordinate pairs per wave");

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// grid: x = q block + n_qb * KV head, y = split, z = sequence; kPfThreads threads
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache, const int64_t* __restrict__ seq_byte_off,
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ n_qtok, int max_q, int64_t max_len,
    int64_t capacity,
    const uint8_t* __restrict__ k_bits, const float* __restrict__ k_sigma, const float* __restrict__ v_sigma,
    float scale_log2, int n_q_heads, int g, int pairing, int sk_bytes, int v_bits, int n_qb, int n_split,
    float* __restrict__ ws, float* __restrict__ out) {
    __shared__ PfSmem sm;
    const int qb = blockIdx.x % n_qb, kvh = blockIdx.x / n_qb, split = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    const int qt = kPfRows / g;  // query tokens per workgroup
    // (out-of-contract values are clamped so that every read stays in the region)
    const int64_t q0 = min(max((int64_t)q_start[s], (int64_t)0), max_len);
    const int nq = (int)min(max((int64_t)n_qtok[s], (int64_t)0), min((int64_t)max_q, max_len - q0));
    const int j0 = qb * qt;
    const int jend = min(j0 + qt, nq);                      // valid tokens [j0, jend)
    const int64_t kend = jend > j0 ? q0 + jend : 0;         // slots any row reads (<= max_len)
    const int64_t n_tiles = (kend + kTile - 1) / kTile;
    const int64_t t0 = n_tiles * split / n_split, t1 = n_tiles * (split + 1) / n_split;

    const int SK = sk_bytes, KB = kTile * SK;
    const int VR = kHeadDim * 8 * v_bits;  // V runs
    const int TB = KB + VR + 2 * kTile * 4;
    const int n_chunks = TB / 16;
    const uint8_t* head_base = cache + seq_byte_off[s] + (int64_t)kvh * (capacity / kTile) * TB;
    auto dma_tile = [&](int64_t tau, int buf) {
        const uint8_t* src = head_base + tau * TB;
        const uint32_t base = (uint32_t)(uintptr_t)(lds_u8*)sm.stage[buf];
#pragma unroll
        for (int k = 0; k < kPfDmaPerThread; ++k) {
            const int ch0 = (kPfWaves * k + wave) * 64, ch = ch0 + lane;
            if (ch0 < n_chunks && ch < n_chunks) dma16(src + 16 * ch, base + 16 * ch0);
        }
    };

    // ---------------------------------------------------------------- prologue
    // this thread's row (the lane's QK/PV column) and its position
    const int r = 32 * wave + col;
    const int rj = j0 + r / g, rh = r % g;
    const bool row_exists = r < qt * g && rj < max_q;
    const bool row_valid = row_exists && rj < nq;
    const int64_t rpos = q0 + rj;
    // blocks: lane = block index b, its width; K order = widths descending, index ascending
    const int my_w = k_bits[kvh * kMaxBlocks + lane];
    const float my_ks = k_sigma[kvh * kMaxBlocks + lane];
    int my_pos = 0, my_koff = 0, n_fields = 0;
    {
        const unsigned long long below = (1ull << lane) - 1ull;
        int bits = 0, nf = 0;
#pragma unroll
        for (int w = 16; w >= 1; --w) {
            if (w > 8 && w < 16) continue;
            const unsigned long long mk = __ballot(my_w == w);
            if (my_w == w) {
                my_pos = nf + 2 * __popcll(mk & below);
                my_koff = bits + 2 * w * __popcll(mk & below);
            }
            bits += 2 * w * __popcll(mk);
            nf += 2 * __popcll(mk);
        }
        n_fields = nf;
    }
    // passthrough widths: K16 (every block 16 bits: 256-byte records) and V16
    const bool k16 = sk_bytes == 16 * kMaxBlocks * 2 / 8, v16 = v_bits == 16;
    const int cp = pairing == KVQ_PAIR_HALF ? lane : 2 * lane;
    const int cq = pairing == KVQ_PAIR_HALF ? lane + kMaxBlocks : 2 * lane + 1;
    if (wave == 0) {
        if (my_w > 0) {
            sm.fcoord[my_pos] = (uint8_t)cp;
            sm.fcoord[my_pos + 1] = (uint8_t)cq;
            const float f = k16 ? scale_log2 : my_ks * scale_log2;  // passthrough: the raw value, no sigma
            sm.fsig[my_pos] = f;
            sm.fsig[my_pos + 1] = f;
        }
        if (2 * lane >= n_fields) {
            sm.fcoord[2 * lane] = 0; sm.fcoord[2 * lane + 1] = 0;
            sm.fsig[2 * lane] = 0.f; sm.fsig[2 * lane + 1] = 0.f;
        }
    } else if (wave == 1) {
        const float vs = v16 ? 1.f : v_sigma[kvh * kMaxBlocks + lane];
        sm.vsig[cp] = vs;
        sm.vsig[cq] = vs;
    }
    for (int i = tid; i < 510; i += kPfThreads) sm.lev[i] = c_levels[i];
    const bool vpairs = v_bits <= 5;
    if (vpairs)
        for (int e = tid; e < (1 << (2 * v_bits)); e += kPfThreads)
            sm.vpair[e] = (uint32_t)c_levels[KVQ_CB_OFF(v_bits) + (e & ((1 << v_bits) - 1))] |
                          ((uint32_t)c_levels[KVQ_CB_OFF(v_bits) + (e >> v_bits)] << 16);
    // the workgroup's query rows, binary16 [rows][128], over the tile buffers (zero rows
    // where no valid query is)
    {
        uint4* qs = (uint4*)sm.stage;
        for (int i = tid; i < kPfRows * kHeadDim / 8; i += kPfThreads) {
            const int rr = i >> 4, part = i & 15;
            const int jj = j0 + rr / g, hh = rr % g;
            uint4 v = uint4{0, 0, 0, 0};
            if (rr < qt * g && jj < nq)
                v = ((const uint4*)(q + (((int64_t)s * max_q + jj) * n_q_heads + (int64_t)kvh * g + hh) * kHeadDim))[part];
            qs[i] = v;
        }
    }
    __syncthreads();
    // B operands of QK: lane (h, col) holds K-order positions 16 ks + 8 h + i of row r
    uint32_t qh[8][4], ql[8][4];
    {
        const uint16_t* qrow = (const uint16_t*)sm.stage + r * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const int f = 16 * ks + 8 * h + i;
                const float a = h2f(qrow[sm.fcoord[f]]) * sm.fsig[f];
                const float b = h2f(qrow[sm.fcoord[f + 1]]) * sm.fsig[f + 1];
                const _Float16 ah = (_Float16)a, bh = (_Float16)b;
                qh[ks][i / 2] = (uint32_t)__builtin_bit_cast(uint16_t, ah) | ((uint32_t)__builtin_bit_cast(uint16_t, bh) << 16);
                ql[ks][i / 2] = pack_h2(a - (float)ah, b - (float)bh);
            }
    }
    __syncthreads();  // the staged queries are consumed: the tile area is free
    if (t0 < t1) dma_tile(t0, 0);
    // K-order positions past the fields stay zero in every dequantized K row
    for (int i = tid; i < kTile * (kHeadDim / 2); i += kPfThreads) {
        const int t = i >> 6, pp = 2 * (i & 63);
        if (pp >= n_fields) *(uint32_t*)&sm.kd[t * kPfKS + pp] = 0u;
    }

    // per-lane dequantization constants
    const int kw = my_w, kcb = 2 * KVQ_CB_OFF(kw > 0 && kw <= 8 ? kw : 1);  // byte offset of the width's levels
    const uint32_t kmask = kw > 0 && kw <= 8 ? (1u << kw) - 1u : 0u;
    const int kword = my_koff >> 5, kshift = my_koff & 31;
    const int sp = lane & 31, vpar = lane >> 5;                  // V: slots 2sp, 2sp+1; coordinate parity
    const int vbit = 2 * sp * v_bits, vword = vbit >> 5, vshift = vbit & 31;
    const uint32_t vmask = v16 ? 0xffffu : (1u << v_bits) - 1u, vmask2 = vpairs ? (1u << (2 * v_bits)) - 1u : 0u;
    const int vcb = 2 * KVQ_CB_OFF(v16 ? 1 : v_bits);

    floatx16 o[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[cb][i] = 0.f;
    float mref = -INFINITY, lrun = 0.f;
    float vexp = 0.f, vlim = (float)(1 << kVNormExp);  // the reference's power of two e, and 2^(7+e)

    for (int64_t tau = t0; tau < t1; ++tau) {
        const int buf = (int)((tau - t0) & 1);
        __builtin_amdgcn_s_waitcnt(wait_vm(0));  // this wave's part of tile tau has landed
        __syncthreads();                         // ... every wave's; the other buffer is free
        if (tau + 1 < t1) dma_tile(tau + 1, buf ^ 1);
        const uint8_t* st = sm.stage[buf];
        // ---- dequantize K: wave w keys [KPW w, KPW (w+1)), lane = block (two fields);
        // eight keys at a time, every read of a batch issued before the first use
        constexpr int KPW = kTile / kPfWaves, CPW = kHeadDim / kPfWaves;
        if (kw > 0) {
#pragma unroll
            for (int i0 = 0; i0 < KPW; i0 += 8) {
                uint32_t lo[8], hi[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t* rec = (const uint32_t*)(st + (KPW * wave + i0 + i) * SK);
                    lo[i] = rec[kword];
                    hi[i] = rec[kword + 1];
                }
                uint32_t lk[8];
                if (k16) {  // the block's two raw binary16 values are one record word
#pragma unroll
                    for (int i = 0; i < 8; ++i) lk[i] = lo[i];
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t x = alignbit(hi[i], lo[i], kshift);
                        lk[i] = lds_u16(sm.lev, kcb + 2 * (x & kmask)) | (lds_u16(sm.lev, kcb + 2 * ((x >> kw) & kmask)) << 16);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) *(uint32_t*)&sm.kd[(KPW * wave + i0 + i) * kPfKS + my_pos] = lk[i];
            }
        }
        // ---- dequantize V: wave w coordinates [CPW w, CPW (w+1)), lane = (slot pair,
        // coordinate parity); one pair lookup per two slots for widths <= 5
        {
            const uint32_t* runs = (const uint32_t*)(st + KB);
#pragma unroll
            for (int i0 = 0; i0 < CPW / 2; i0 += 8) {
                uint32_t lo[8], hi[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t* run = runs + (CPW * wave + 2 * (i0 + i) + vpar) * 2 * v_bits;
                    lo[i] = run[vword];
                    hi[i] = run[vword + 1];
                }
                uint32_t lv[8];
                if (v16) {  // two slots' raw binary16 values are one run word
#pragma unroll
                    for (int i = 0; i < 8; ++i) lv[i] = lo[i];
                } else if (vpairs) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) lv[i] = lds_u32(sm.vpair, 4 * (alignbit(hi[i], lo[i], vshift) & vmask2));
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t x = alignbit(hi[i], lo[i], vshift);
                        lv[i] = lds_u16(sm.lev, vcb + 2 * (x & vmask)) | (lds_u16(sm.lev, vcb + 2 * ((x >> v_bits) & vmask)) << 16);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) *(uint32_t*)&sm.vd[(CPW * wave + 2 * (i0 + i) + vpar) * kPfVS + 2 * sp] = lv[i];
            }
        }
        __syncthreads();
        // ---- per 32-key half kb of the tile: QK (S^T, this wave's 32 rows), softmax, PV
        const float* skl = (const float*)(st + KB + VR);
        const float* svl = skl + kTile;
        const int64_t key0 = tau * kTile;
        // keys of this tile the row may see: index <= lim (-1: none)
        const int lim = row_valid ? (int)min(max(rpos - key0, (int64_t)-1), (int64_t)kTile) : -1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            floatx16 acc;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                H8 a, bh, bl;
                const uint4 a4 = *(const uint4*)&sm.kd[(32 * kb + col) * kPfKS + 16 * ks + 8 * h];
                a.u[0] = a4.x; a.u[1] = a4.y; a.u[2] = a4.z; a.u[3] = a4.w;
#pragma unroll
                for (int u = 0; u < 4; ++u) { bh.u[u] = qh[ks][u]; bl.u[u] = ql[ks][u]; }
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.h, bh.h, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.h, bl.h, acc, 0, 0, 0);
            }
            // logits: element i is key 32 kb + 8 (i/4) + 4 h + i%4
            const bool need_mask = lim < 32 * kb + 31;
            float tm = -INFINITY;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int kk = 32 * kb + 8 * jj + 4 * h;
                const float4 sc = k16 ? float4{1.f, 1.f, 1.f, 1.f} : *(const float4*)(skl + kk);
                acc[4 * jj + 0] *= sc.x; acc[4 * jj + 1] *= sc.y;
                acc[4 * jj + 2] *= sc.z; acc[4 * jj + 3] *= sc.w;
                if (need_mask) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (kk + e > lim) acc[4 * jj + e] = -INFINITY;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) tm = fmaxf(tm, acc[4 * jj + e]);
            }
            tm = xor32_max(tm);
            float svv[4][4];  // this lane's keys' value norms (1 for the V16 passthrough)
            float smax = 0.f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float4 sv = v16 ? float4{1.f, 1.f, 1.f, 1.f} : *(const float4*)(svl + 32 * kb + 8 * jj + 4 * h);
                svv[jj][0] = sv.x; svv[jj][1] = sv.y; svv[jj][2] = sv.z; svv[jj][3] = sv.w;
                smax = fmaxf(smax, fmaxf(fmaxf(sv.x, sv.y), fmaxf(sv.z, sv.w)));
            }
            if (__ballot(tm > mref + kPfSlack || smax > vlim)) {
                // the half tile's largest value norm (both lanes' keys) sets the power of two
                const float vnew = fmaxf(vexp, (float)(__builtin_amdgcn_frexp_expf(xor32_max(smax)) - kVNormExp));
                const float mnew = fmaxf(mref, tm);
                const float alpha =
                    mref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mref + vexp) - (mnew + vnew));
                mref = mnew;
                vexp = vnew;
                vlim = __builtin_amdgcn_ldexpf(1.f, kVNormExp + (int)vnew);
                lrun *= alpha;
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[cb][i] *= alpha;
            }
            const float mb = mref == -INFINITY ? 0.f : mref + vexp;  // rows that have seen nothing keep p = 0
            float psum = 0.f;
            uint32_t ph[8], pl[8];  // P' (p s^V 2^-e) as binary16 hi + lo pairs in the accumulator's key order
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = __builtin_amdgcn_exp2f(acc[4 * jj + e] - mb);
                    psum += p;
                    pv[e] = p * svv[jj][e];
                }
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    const _Float16 a = (_Float16)pv[e], b = (_Float16)pv[e + 1];
                    ph[2 * jj + e / 2] = (uint32_t)__builtin_bit_cast(uint16_t, a) |
                                         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
                    pl[2 * jj + e / 2] = pack_h2(pv[e] - (float)a, pv[e + 1] - (float)b);
                }
            }
            lrun += psum;
            // PV: MFMA m takes keys 32 kb + 16 m + 8 (i/4) + 4 h + i%4, i = 0..7
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                H8 bh, bl;
#pragma unroll
                for (int u = 0; u < 4; ++u) { bh.u[u] = ph[4 * m + u]; bl.u[u] = pl[4 * m + u]; }
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const uint16_t* vrow = &sm.vd[(32 * cb + col) * kPfVS + 32 * kb + 16 * m + 4 * h];
                    const uint2 v0 = *(const uint2*)vrow;
                    const uint2 v1 = *(const uint2*)(vrow + 8);
                    H8 a;
                    a.u[0] = v0.x; a.u[1] = v0.y; a.u[2] = v1.x; a.u[3] = v1.y;
                    o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.h, bh.h, o[cb], 0, 0, 0);
                    o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a.h, bl.h, o[cb], 0, 0, 0);
                }
            }
        }
    }

    // ---------------------------------------------------------------- epilogue
    // lanes l and l ^ 32 hold the same row (different keys, then different coordinates)
    const float lsum = xor32_sum(lrun);
    if (!row_exists) return;
    const int64_t orow = ((int64_t)s * max_q + rj) * n_q_heads + (int64_t)kvh * g + rh;
    if (n_split == 1) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        float* dst = out + orow * kHeadDim;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int c = 32 * cb + 8 * jj + 4 * h;
                const float4 vs = *(const float4*)&sm.vsig[c];
                *(float4*)(dst + c) = float4{o[cb][4 * jj] * vs.x * inv, o[cb][4 * jj + 1] * vs.y * inv,
                                             o[cb][4 * jj + 2] * vs.z * inv, o[cb][4 * jj + 3] * vs.w * inv};
            }
    } else {
        float* part = ws + (orow * n_split + split) * (kHeadDim + 2);
        if (h == 0) { part[0] = mref == -INFINITY ? mref : mref + vexp; part[1] = lsum; }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int c = 32 * cb + 8 * jj + 4 * h;
                const float4 vs = *(const float4*)&sm.vsig[c];
                *(float2*)(part + 2 + c) = float2{o[cb][4 * jj] * vs.x, o[cb][4 * jj + 1] * vs.y};
                *(float2*)(part + 4 + c) = float2{o[cb][4 * jj + 2] * vs.z, o[cb][4 * jj + 3] * vs.w};
            }
    }
}

int plan_prefill(const kvq_geom& g, int n_q_heads, int n_seq, int max_q, int64_t max_len, int n_split_req,
                 PrefillPlan* plan) {
    const int grp = n_q_heads / g.n_kv_heads;
    if (g.head_dim != kHeadDim || grp > kPfMaxGroup) return KVQ_ERR_SHAPE;
    const int qt = kPfRows / grp;
    plan->n_qb = (max_q + qt - 1) / qt;
    const int64_t max_tiles = (max_len + kTile - 1) / kTile;
    int n_split = n_split_req;
    if (n_split <= 0) {
        static int slots = 0;
        if (slots == 0) {
            int dev = 0, cus = 0, occ = 0;
            if (hipGetDevice(&dev) == hipSuccess &&
                hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, prefill_kernel, kPfThreads, 0) == hipSuccess && occ > 0)
                slots = cus * occ;
            else
                slots = 512;
        }
        const int64_t base = (int64_t)plan->n_qb * g.n_kv_heads * (n_seq > 0 ? n_seq : 1);
        int64_t want = (slots + base - 1) / (base > 0 ? base : 1);
        const int64_t cap = max_tiles / 8 > 1 ? max_tiles / 8 : 1;  // at least 8 tiles per split
        if (want > cap) want = cap;
        if (want < 1) want = 1;
        n_split = (int)want;
    }
    if (n_split > 65535) return KVQ_ERR_ARG;
    plan->n_split = n_split;
    plan->workspace = n_split > 1 ? (int64_t)n_seq * max_q * n_q_heads * n_split * (kHeadDim + 2) * 4 : 0;
    return KVQ_OK;
}

hipError_t launch_prefill(const kvq_geom& g, const PrefillPlan& plan, int n_q_heads, const uint16_t* q,
                          const uint8_t* cache, const int64_t* seq_byte_off, const int32_t* q_start,
                          const int32_t* n_q, int n_seq, int max_q, int64_t max_len, const uint8_t* k_bits, const float* k_sigma,
                          const float* v_sigma, float softmax_scale, float* out, float* ws, hipStream_t st) {
    const int grp = n_q_heads / g.n_kv_heads;
    dim3 grid(plan.n_qb * g.n_kv_heads, plan.n_split, n_seq);
    hipLaunchKernelGGL(prefill_kernel, grid, dim3(kPfThreads), 0, st, q, cache, seq_byte_off, q_start, n_q, max_q,
                       max_len, g.capacity_tokens, k_bits, k_sigma, v_sigma, softmax_scale * kLog2e, n_q_heads, grp,
                       g.rope_pairing, (int)k_record_bytes(g.k_budget), g.v_bits, plan.n_qb, plan.n_split, ws, out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.n_split == 1) return e;
    return launch_merge(n_seq * max_q * n_q_heads, plan.n_split, ws, out, st);
}

}  // namespace kvq
