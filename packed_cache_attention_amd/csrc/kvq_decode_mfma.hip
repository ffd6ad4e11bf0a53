// kvq_decode_mfma.hip -- dispatch of the matrix-core decode kernel on the value
// width; the kernel itself is in kvq_decode_mfma.h and its instantiations in
// kvq_decode_mfma_v1.hip .. kvq_decode_mfma_v8.hip and kvq_decode_mfma_v16.hip
// (compiled in parallel).
#include "kvq_internal.h"

namespace kvq {

template <int V>
hipError_t launch_mfma_v(const kvq_geom& g, const DecodePlan& plan, int n_q_heads, const uint16_t* q,
                         uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len, int n_seq,
                         int64_t max_len, const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                         float scale_log2, float* partials, hipStream_t st, const AppendArgs& app);
#define KVQ_EXTERN(VB) extern template hipError_t launch_mfma_v<VB>(const kvq_geom&, const DecodePlan&, int,      \
    const uint16_t*, uint8_t*, const int64_t*, const int32_t*, int, int64_t, const uint8_t*, const float*,         \
    const float*, float, float*, hipStream_t, const AppendArgs&);
KVQ_EXTERN(1) KVQ_EXTERN(2) KVQ_EXTERN(3) KVQ_EXTERN(4) KVQ_EXTERN(5) KVQ_EXTERN(6) KVQ_EXTERN(7) KVQ_EXTERN(8)
KVQ_EXTERN(16)
#undef KVQ_EXTERN
template <int V>
int mfma_blocks_per_cu_v(const kvq_geom& g);
#define KVQ_EXTERN(VB) extern template int mfma_blocks_per_cu_v<VB>(const kvq_geom&);
KVQ_EXTERN(1) KVQ_EXTERN(2) KVQ_EXTERN(3) KVQ_EXTERN(4) KVQ_EXTERN(5) KVQ_EXTERN(6) KVQ_EXTERN(7) KVQ_EXTERN(8)
KVQ_EXTERN(16)
#undef KVQ_EXTERN

int mfma_blocks_per_cu(const kvq_geom& g) {
    switch (g.v_bits) {
        case 1: return mfma_blocks_per_cu_v<1>(g);
        case 2: return mfma_blocks_per_cu_v<2>(g);
        case 3: return mfma_blocks_per_cu_v<3>(g);
        case 4: return mfma_blocks_per_cu_v<4>(g);
        case 5: return mfma_blocks_per_cu_v<5>(g);
        case 6: return mfma_blocks_per_cu_v<6>(g);
        case 7: return mfma_blocks_per_cu_v<7>(g);
        case 8: return mfma_blocks_per_cu_v<8>(g);
        case 16: return mfma_blocks_per_cu_v<16>(g);
        default: return 0;
    }
}

hipError_t launch_decode_mfma(const kvq_geom& g, const DecodePlan& plan, int n_q_heads, const uint16_t* q,
                              uint8_t* cache, const int64_t* seq_byte_off, const int32_t* seq_len, int n_seq,
                              int64_t max_len, const uint8_t* k_bits, const float* k_sigma, const float* v_sigma,
                              float scale_log2, float* partials, hipStream_t st, const AppendArgs& app) {
    switch (g.v_bits) {
#define KVQ_CASE(VB)                                                                                            \
    case VB:                                                                                                    \
        return launch_mfma_v<VB>(g, plan, n_q_heads, q, cache, seq_byte_off, seq_len, n_seq, max_len, k_bits,  \
                                 k_sigma, v_sigma, scale_log2, partials, st, app);
        KVQ_CASE(1) KVQ_CASE(2) KVQ_CASE(3) KVQ_CASE(4) KVQ_CASE(5) KVQ_CASE(6) KVQ_CASE(7) KVQ_CASE(8)
        KVQ_CASE(16)
#undef KVQ_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kvq
