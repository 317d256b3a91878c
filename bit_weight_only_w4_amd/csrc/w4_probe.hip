// Bandwidth ceiling probes: a read-only streaming kernel and a copy kernel, both with 128-bit
// accesses and a grid-stride loop.  They give the measured HBM ceiling that the GEMV is compared
// with (My Triton Kernel Ties bitsandbytes, "The roofline first": a measured copy bandwidth rather
// than the spec sheet; Do Quantization and Sparsity make LLM Inference Faster?, "What we did": a
// measured streaming-read ceiling).
#include "w4_common.h"

namespace w4 {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ void __launch_bounds__(kProbeThreads) probe_read_kernel(const uint4* __restrict__ src,
                                                                    int64_t n16,
                                                                    uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = blockIdx.x * (int64_t)kProbeThreads + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = load_stream16(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

__global__ void __launch_bounds__(kProbeThreads) probe_copy_kernel(const uint4* __restrict__ src,
                                                                    uint4* __restrict__ dst,
                                                                    int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  for (int64_t i = blockIdx.x * (int64_t)kProbeThreads + threadIdx.x; i < n16; i += stride) {
    dst[i] = src[i];
  }
}

}  // namespace

hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int blocks = device_cu_count() * 8;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(kProbeThreads), 0, s,
                     reinterpret_cast<const uint4*>(src), n16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int blocks = device_cu_count() * 8;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks), dim3(kProbeThreads), 0, s,
                     reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace w4
