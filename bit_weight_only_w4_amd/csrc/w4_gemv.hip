// Format dispatch of the fused GEMV, the fixed-order split-K reduction, and the static split-K
// scratch of the no-allocation entry point.
#include <mutex>

#include "w4_common.h"

namespace w4 {

// Split-K partials of w4_matmul_splitk_noalloc: a file-scope device array, so that the call needs
// no allocation.  Every device the library runs on holds its own copy (W4_NOALLOC_SCRATCH_BYTES)
// until the process ends; all calls on one device share it, which is why calls that overlap in
// time on one device race.  Host code never passes `scratch` itself to a kernel (on the host the
// name is a stand-in, not a device address): it passes the address hipGetSymbolAddress reports
// for the current device.
static __device__ __align__(256) float scratch[W4_NOALLOC_SCRATCH_BYTES / 4];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_addr[64] = {};
}  // namespace

hipError_t splitk_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device's copy, with it current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

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
