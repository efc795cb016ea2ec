// decode_mfma.hip - bf16 matrix-core decode kernel (not yet enabled).
#include "think_common.h"

namespace thinkkv {

bool mfma_decode_supported(const think_dims&, int) { return false; }
int mfma_decode_chunk(const think_dims&, int) { return 256; }
hipError_t launch_decode_mfma(const think_dims&, const DecodeGeom&, const void*, const void*,
                              const void*, const int32_t*, const int32_t*, int, float, float*,
                              hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace thinkkv
