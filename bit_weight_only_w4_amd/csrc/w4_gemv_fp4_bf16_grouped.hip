// Instantiation of the fused GEMV for one weight x activation format (fp4_bf16), several members
// per launch.
#include "w4_gemv_impl.h"

namespace w4 {
hipError_t launch_gemv_fp4_bf16_grouped(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                        hipStream_t s) {
  return launch_fx<kFP4, kBF16, true>(b, a, groups, p, s);
}
}  // namespace w4
