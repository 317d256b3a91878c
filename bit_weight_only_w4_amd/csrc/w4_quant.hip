// Offline quantizers: fp32 weights -> packed nibbles + per-block scales, decided in fp64.
//
// NF4 (LLM Quantization on RTX 4060: Where 4-bit Decode Falls Behind FP16, "Standard Expectation
// from Quantization"): blocks of 64 along K, absmax A stored as fp32, nibble = nearest code to
// w / A.  The decision compares the fp64 quotient w / A with the fp64 midpoints of neighbouring
// codes: a non-zero gap between the exact ratio and a midpoint is far larger than the fp64
// quotient's rounding error, and an exact tie yields the midpoint itself, which goes to the lower
// index.  An fp32 quotient is not enough: it flips a few nibbles per billion weights.
//
// INT4 (My Triton Kernel Ties bitsandbytes, "The kernels": +8 zero point; LLM Compressor 0.14,
// "Details worth knowing": rint): groups of 128, s = bf16_RNE(fp32(A / 7)), q = clamp(rint(w / s),
// -8, 7) against the rounded s, nibble = q + 8.  fp32(A / 7) is taken as the fp64 quotient rounded
// to fp32, which equals the correctly rounded fp32 quotient (53 >= 2 * 24 + 2).
//
// Asymmetric INT4 (LLM Compressor 0.14, "The fused kernel": a code is the clamped, rounded sum
// of the scale quotient and the zero point; "Details worth knowing": rint): groups of 128,
// lo = min(min w, 0), hi = max(max w, 0), s = bf16_RNE(fp32(fp32(hi - lo) / 15)), z = clamp(rint(-lo / s), 0, 15),
// q = rint(clamp(w / s + z, 0, 15)), quotients in fp64 against the rounded s; the group's word is
// the bf16 bits of s | z << 16.
//
// FP4 (LLM Compressor 0.14, "Details worth knowing": rounding onto the magnitudes
// {0, 0.5, 1, 1.5, 2, 3, 4, 6} by threshold comparisons whose <= and < alternate, exact ties
// landing on even codes): blocks of
// 64, s = fp32(A / 6) (the fp64 quotient rounded to fp32, as for INT4), magnitude index = the
// ladder applied to the fp64 quotient |w| / s, sign bit = (w < 0); the thresholds are dyadic, so
// the fp64 quotient of two fp32 values is on the same side of each as the exact ratio.
//
// One lane handles one pair of weights (one output byte): element 2i goes to the high nibble.
// Absmax is an integer max over |bits| (the order of non-negative floats), reduced across the 32
// lanes of an NF4 block or the 64 lanes of an INT4 group with cross-lane shuffles (asymmetric
// INT4: fp32 min and max the same way).
#include "w4_common.h"

namespace w4 {

// Set to a non-zero value by a quantize kernel that meets a NaN or Inf weight.  Reset and read
// back by the host around every quantize call.
__device__ int g_w4_nonfinite;

namespace {

__constant__ uint32_t c_nf4_code_bits[16] = W4_NF4_CODE_BITS;

__device__ inline uint32_t nf4_index(double r, const double (&mid)[15]) {
  uint32_t idx = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) idx += (r > mid[i]) ? 1u : 0u;
  return idx;
}

__global__ void __launch_bounds__(256) quant_nf4_kernel(const float* __restrict__ w, int64_t pairs,
                                                         uint8_t* __restrict__ packed,
                                                         float* __restrict__ absmax) {
  const int64_t p = blockIdx.x * 256ll + threadIdx.x;
  const bool valid = p < pairs;  // pairs is a multiple of 32: a whole block is valid or not
  const float2 v = reinterpret_cast<const float2*>(w)[valid ? p : 0];
  const uint32_t a0 = __float_as_uint(v.x) & 0x7FFFFFFFu;
  const uint32_t a1 = __float_as_uint(v.y) & 0x7FFFFFFFu;
  if (valid && (a0 >= 0x7F800000u || a1 >= 0x7F800000u)) g_w4_nonfinite = 1;
  uint32_t m = a0 > a1 ? a0 : a1;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)m, off);
    m = o > m ? o : m;
  }
  const float amax = __uint_as_float(m);
  uint32_t i0 = 7, i1 = 7;
  if (m != 0) {
    double mid[15];
#pragma unroll
    for (int i = 0; i < 15; ++i) {
      mid[i] = ((double)__uint_as_float(c_nf4_code_bits[i]) +
                (double)__uint_as_float(c_nf4_code_bits[i + 1])) * 0.5;
    }
    const double a = (double)amax;
    i0 = nf4_index((double)v.x / a, mid);
    i1 = nf4_index((double)v.y / a, mid);
  }
  if (valid) {
    packed[p] = (uint8_t)((i0 << 4) | i1);
    if ((threadIdx.x & 31) == 0) absmax[p >> 5] = amax;
  }
}

__global__ void __launch_bounds__(256) quant_int4_kernel(const float* __restrict__ w, int64_t pairs,
                                                          uint8_t* __restrict__ packed,
                                                          uint16_t* __restrict__ scale) {
  const int64_t p = blockIdx.x * 256ll + threadIdx.x;
  const bool valid = p < pairs;  // pairs is a multiple of 64: a whole group is valid or not
  const float2 v = reinterpret_cast<const float2*>(w)[valid ? p : 0];
  const uint32_t a0 = __float_as_uint(v.x) & 0x7FFFFFFFu;
  const uint32_t a1 = __float_as_uint(v.y) & 0x7FFFFFFFu;
  if (valid && (a0 >= 0x7F800000u || a1 >= 0x7F800000u)) g_w4_nonfinite = 1;
  uint32_t m = a0 > a1 ? a0 : a1;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)m, off);
    m = o > m ? o : m;
  }
  const float s32 = (float)((double)__uint_as_float(m) / 7.0);
  const uint32_t u = __float_as_uint(s32);
  const uint32_t sb = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // bf16, nearest even
  const double s = (double)__uint_as_float(sb << 16);
  uint32_t n0 = 8, n1 = 8;
  if (s != 0.0) {
    double q0 = rint((double)v.x / s), q1 = rint((double)v.y / s);
    q0 = q0 < -8.0 ? -8.0 : (q0 > 7.0 ? 7.0 : q0);
    q1 = q1 < -8.0 ? -8.0 : (q1 > 7.0 ? 7.0 : q1);
    n0 = (uint32_t)((int)q0 + 8);
    n1 = (uint32_t)((int)q1 + 8);
  }
  if (valid) {
    packed[p] = (uint8_t)((n0 << 4) | n1);
    if ((threadIdx.x & 63) == 0) scale[p >> 6] = (uint16_t)sb;
  }
}

__global__ void __launch_bounds__(256) quant_int4_asym_kernel(const float* __restrict__ w,
                                                               int64_t pairs,
                                                               uint8_t* __restrict__ packed,
                                                               uint32_t* __restrict__ words) {
  const int64_t p = blockIdx.x * 256ll + threadIdx.x;
  const bool valid = p < pairs;  // pairs is a multiple of 64: a whole group is valid or not
  const float2 v = reinterpret_cast<const float2*>(w)[valid ? p : 0];
  const uint32_t a0 = __float_as_uint(v.x) & 0x7FFFFFFFu;
  const uint32_t a1 = __float_as_uint(v.y) & 0x7FFFFFFFu;
  if (valid && (a0 >= 0x7F800000u || a1 >= 0x7F800000u)) g_w4_nonfinite = 1;
  // the range with 0 in it: lo <= 0 <= hi
  float lo = fminf(fminf(v.x, v.y), 0.0f), hi = fmaxf(fmaxf(v.x, v.y), 0.0f);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    lo = fminf(lo, __shfl_xor(lo, off));
    hi = fmaxf(hi, __shfl_xor(hi, off));
  }
  const float span = hi - lo;  // one IEEE fp32 subtraction
  const float s32 = (float)((double)span / 15.0);
  const uint32_t u = __float_as_uint(s32);
  const uint32_t sb = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // bf16, nearest even
  const double s = (double)__uint_as_float(sb << 16);
  uint32_t n0 = 0, n1 = 0, z = 0;
  if (s != 0.0) {
    double zf = rint(-(double)lo / s);
    zf = zf < 0.0 ? 0.0 : (zf > 15.0 ? 15.0 : zf);
    z = (uint32_t)zf;
    double q0 = (double)v.x / s + zf, q1 = (double)v.y / s + zf;  // w / s + z
    q0 = rint(q0 < 0.0 ? 0.0 : (q0 > 15.0 ? 15.0 : q0));        // clamp, round
    q1 = rint(q1 < 0.0 ? 0.0 : (q1 > 15.0 ? 15.0 : q1));
    n0 = (uint32_t)q0;
    n1 = (uint32_t)q1;
  }
  if (valid) {
    packed[p] = (uint8_t)((n0 << 4) | n1);
    if ((threadIdx.x & 63) == 0) words[p >> 6] = sb | (z << 16);
  }
}

// FP4 magnitude index of y = |w| / s >= 0: one step past each threshold crossed; a value on
// 0.25, 1.25, 2.5 or 5 stays below, one on 0.75, 1.75 or 3.5 goes above (the even index).
__device__ inline uint32_t fp4_magnitude(double y) {
  return (y > 0.25 ? 1u : 0u) + (y >= 0.75 ? 1u : 0u) + (y > 1.25 ? 1u : 0u) + (y >= 1.75 ? 1u : 0u) +
         (y > 2.5 ? 1u : 0u) + (y >= 3.5 ? 1u : 0u) + (y > 5.0 ? 1u : 0u);
}

__global__ void __launch_bounds__(256) quant_fp4_kernel(const float* __restrict__ w, int64_t pairs,
                                                         uint8_t* __restrict__ packed,
                                                         float* __restrict__ scale) {
  const int64_t p = blockIdx.x * 256ll + threadIdx.x;
  const bool valid = p < pairs;  // pairs is a multiple of 32: a whole block is valid or not
  const float2 v = reinterpret_cast<const float2*>(w)[valid ? p : 0];
  const uint32_t a0 = __float_as_uint(v.x) & 0x7FFFFFFFu;
  const uint32_t a1 = __float_as_uint(v.y) & 0x7FFFFFFFu;
  if (valid && (a0 >= 0x7F800000u || a1 >= 0x7F800000u)) g_w4_nonfinite = 1;
  uint32_t m = a0 > a1 ? a0 : a1;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)m, off);
    m = o > m ? o : m;
  }
  const float s32 = (float)((double)__uint_as_float(m) / 6.0);
  const double s = (double)s32;
  uint32_t n0 = 0, n1 = 0;
  if (s != 0.0) {
    n0 = fp4_magnitude(fabs((double)v.x) / s) | (v.x < 0.0f ? 8u : 0u);
    n1 = fp4_magnitude(fabs((double)v.y) / s) | (v.y < 0.0f ? 8u : 0u);
  }
  if (valid) {
    packed[p] = (uint8_t)((n0 << 4) | n1);
    if ((threadIdx.x & 31) == 0) scale[p >> 5] = s32;
  }
}

}  // namespace

hipError_t quantize_error_reset(hipStream_t s) {
  const int zero = 0;
  return hipMemcpyToSymbolAsync(HIP_SYMBOL(g_w4_nonfinite), &zero, sizeof(int), 0,
                                hipMemcpyHostToDevice, s);
}

hipError_t quantize_error_read(int* flag, hipStream_t s) {
  hipError_t e = hipMemcpyFromSymbolAsync(flag, HIP_SYMBOL(g_w4_nonfinite), sizeof(int), 0,
                                          hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

hipError_t launch_quantize_nf4(const float* w, int64_t n, int64_t k, uint8_t* packed,
                               float* absmax, hipStream_t s) {
  const int64_t pairs = n * (k / 2);
  const int64_t blocks = (pairs + 255) / 256;
  hipLaunchKernelGGL(quant_nf4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, pairs, packed,
                     absmax);
  return hipGetLastError();
}

hipError_t launch_quantize_fp4(const float* w, int64_t n, int64_t k, uint8_t* packed, float* scale,
                               hipStream_t s) {
  const int64_t pairs = n * (k / 2);
  const int64_t blocks = (pairs + 255) / 256;
  hipLaunchKernelGGL(quant_fp4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, pairs, packed,
                     scale);
  return hipGetLastError();
}

hipError_t launch_quantize_int4_asym(const float* w, int64_t n, int64_t k, uint8_t* packed,
                                     uint32_t* words, hipStream_t s) {
  const int64_t pairs = n * (k / 2);
  const int64_t blocks = (pairs + 255) / 256;
  hipLaunchKernelGGL(quant_int4_asym_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, pairs,
                     packed, words);
  return hipGetLastError();
}

hipError_t launch_quantize_int4(const float* w, int64_t n, int64_t k, uint8_t* packed,
                                uint16_t* scale, hipStream_t s) {
  const int64_t pairs = n * (k / 2);
  const int64_t blocks = (pairs + 255) / 256;
  hipLaunchKernelGGL(quant_int4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, pairs, packed,
                     scale);
  return hipGetLastError();
}

}  // namespace w4
