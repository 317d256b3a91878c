// Format dispatch of the fused GEMV and the fixed-order split-K reduction.
#include "w4_common.h"

namespace w4 {

hipError_t launch_gemv_nf4_f16(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                               hipStream_t s);
hipError_t launch_gemv_nf4_bf16(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                hipStream_t s);
hipError_t launch_gemv_int4_f16(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                hipStream_t s);
hipError_t launch_gemv_int4_bf16(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                 hipStream_t s);
hipError_t launch_gemv_nf4_f16_grouped(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                       hipStream_t s);
hipError_t launch_gemv_nf4_bf16_grouped(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                        hipStream_t s);
hipError_t launch_gemv_int4_f16_grouped(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                        hipStream_t s);
hipError_t launch_gemv_int4_bf16_grouped(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                         hipStream_t s);
hipError_t launch_gemv_fp4_f16(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                               hipStream_t s);
hipError_t launch_gemv_fp4_bf16(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                hipStream_t s);
hipError_t launch_gemv_fp4_f16_grouped(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                       hipStream_t s);
hipError_t launch_gemv_fp4_bf16_grouped(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                        hipStream_t s);
hipError_t launch_gemv_int4a_f16(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                 hipStream_t s);
hipError_t launch_gemv_int4a_bf16(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                  hipStream_t s);
hipError_t launch_gemv_int4a_f16_grouped(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                         hipStream_t s);
hipError_t launch_gemv_int4a_bf16_grouped(int b, const GemvArgs& a, int groups, const GemvPlan& p,
                                          hipStream_t s);

namespace {

// Split-K second pass: y = sum over splits of the fp32 partials, always in the order s = 0, 1, ...,
// so the result is bitwise reproducible; y is overwritten, never accumulated into.
__global__ void splitk_reduce_kernel(const float* __restrict__ partial, float* __restrict__ y,
                                     int64_t count, int splits) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v = 0.0f;
    for (int s = 0; s < splits; ++s) v += partial[s * count + i];  // fixed order s = 0, 1, ...
    y[i] = v;
  }
}

}  // namespace

hipError_t launch_gemv(int fmt, int b, const GemvArgs& a, int groups, const GemvPlan& p,
                       hipStream_t s) {
  if (groups > 1) {
    switch (fmt) {
      case W4_NF4_X_F16: return launch_gemv_nf4_f16_grouped(b, a, groups, p, s);
      case W4_NF4_X_BF16: return launch_gemv_nf4_bf16_grouped(b, a, groups, p, s);
      case W4_INT4_X_F16: return launch_gemv_int4_f16_grouped(b, a, groups, p, s);
      case W4_INT4_X_BF16: return launch_gemv_int4_bf16_grouped(b, a, groups, p, s);
      case W4_FP4_X_F16: return launch_gemv_fp4_f16_grouped(b, a, groups, p, s);
      case W4_FP4_X_BF16: return launch_gemv_fp4_bf16_grouped(b, a, groups, p, s);
      case W4_INT4A_X_F16: return launch_gemv_int4a_f16_grouped(b, a, groups, p, s);
      case W4_INT4A_X_BF16: return launch_gemv_int4a_bf16_grouped(b, a, groups, p, s);
    }
    return hipErrorInvalidValue;
  }
  switch (fmt) {
    case W4_NF4_X_F16: return launch_gemv_nf4_f16(b, a, groups, p, s);
    case W4_NF4_X_BF16: return launch_gemv_nf4_bf16(b, a, groups, p, s);
    case W4_INT4_X_F16: return launch_gemv_int4_f16(b, a, groups, p, s);
    case W4_INT4_X_BF16: return launch_gemv_int4_bf16(b, a, groups, p, s);
    case W4_FP4_X_F16: return launch_gemv_fp4_f16(b, a, groups, p, s);
    case W4_FP4_X_BF16: return launch_gemv_fp4_bf16(b, a, groups, p, s);
    case W4_INT4A_X_F16: return launch_gemv_int4a_f16(b, a, groups, p, s);
    case W4_INT4A_X_BF16: return launch_gemv_int4a_bf16(b, a, groups, p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_splitk_reduce(const float* partial, float* y, int64_t count, int splits,
                                hipStream_t s) {
  const int threads = 256;
  int64_t blocks = (count + threads - 1) / threads;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(threads), 0, s, partial, y,
                     count, splits);
  return hipGetLastError();
}

}  // namespace w4
