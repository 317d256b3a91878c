// MFMA small-batch path (placeholder until the dequantize-in-LDS kernel lands).
#include "w4_common.h"

namespace w4 {

hipError_t launch_mfma(int, const uint16_t*, const uint8_t*, const void*, int64_t, int64_t,
                       int64_t, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace w4
