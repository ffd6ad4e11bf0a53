// kvq_decode_mfma.hip -- matrix-core decode kernel (not built yet).
#include "kvq_internal.h"

namespace kvq {

hipError_t launch_decode_mfma(const kvq_geom&, const DecodePlan&, int, const uint16_t*, const uint8_t*,
                              const int64_t*, const int32_t*, int, int64_t, const uint8_t*, const float*,
                              const float*, float, float*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace kvq
