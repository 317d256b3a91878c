// Instantiation of the fused GEMV for one weight x activation format (int4a_bf16), several members
// per launch.
#include "w4_gemv_impl.h"

namespace w4 {
hipError_t launch_gemv_int4a_bf16_grouped(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                         hipStream_t s) {
  return launch_fx<kINT4A, kBF16, true>(b, a, groups, p, s);
}
}  // namespace w4
