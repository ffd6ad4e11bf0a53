// kvq_decode_mfma_v16.hip -- matrix-core decode kernels for 16-bit values (the K-only mode).
#include "kvq_decode_mfma.h"

namespace kvq {
template hipError_t launch_mfma_v<16>(const kvq_geom&, const DecodePlan&, int, const uint16_t*, uint8_t*,
                                     const int64_t*, const int32_t*, int, int64_t, const uint8_t*, const float*,
                                     const float*, float, float*, hipStream_t, const AppendArgs&);
template int mfma_blocks_per_cu_v<16>(const kvq_geom&);
}  // namespace kvq
