// Two-pass ablation: dequantize W to fp16 in a workspace, then a dense fp16-weight GEMV/GEMM.
//
// This is the out-of-place path whose byte count the pages call the quantization tax: read 0.5 B,
// write 2 B and read back 2 B per weight, 4.5 B in total against 0.5 B for the fused kernel
// (LLM Quantization on RTX 4060: Where 4-bit Decode Falls Behind FP16, "The Quantization Tax: A
// Byte-Accounting Model"); the first version of the GEMV in My Triton Kernel Ties bitsandbytes
// ("The kernels", v1) works the same way.  It is kept as a measured baseline, not as a product
// path.
//
// The decoded weights are materialized in fp16 for both activation types: for INT4,
// (q - 8) * s is exact in fp16 whenever it is in fp16 range; for INT4A, (q - z) * s has up to
// 12 significant bits and is rounded once to fp16; for NF4 and FP4, code * scale is
// rounded once to fp16 (relative error <= 2^-11, inside the acceptance bound).  bf16 would not be.
#include "w4_common.h"

namespace w4 {
namespace {

__constant__ uint32_t c_nf4_code_bits2[16] = W4_NF4_CODE_BITS;
__constant__ uint32_t c_fp4_code_bits2[16] = W4_FP4_CODE_BITS;

template <int FMT>
__global__ void __launch_bounds__(256) dequant_kernel(const uint4* __restrict__ packed,
                                                       const void* __restrict__ scales,
                                                       int64_t chunks, int cpr, int64_t k,
                                                       uint4* __restrict__ out) {
  for (int64_t c = blockIdx.x * 256ll + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * 256) {
    const int64_t row = c / cpr;
    const int cr = (int)(c - row * cpr);
    float s;
    int zp = 8;  // the stored nibble's offset: 8 (INT4), the group's zero point (INT4A)
    if (FMT == kINT4A) {
      const uint32_t word = reinterpret_cast<const uint32_t*>(scales)[row * (k >> 7) + (cr >> 2)];
      s = __uint_as_float(word << 16);
      zp = (int)((word >> 16) & 15u);
    } else if (!is_g128(FMT)) {
      s = reinterpret_cast<const float*>(scales)[row * (k >> 6) + (cr >> 1)];
    } else {
      s = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(scales)[row * (k >> 7) + (cr >> 2)] << 16);
    }
    const uint4 p = packed[c];
    const uint32_t wv[4] = {p.x, p.y, p.z, p.w};
    uint32_t o[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = (wv[j] >> (8 * b)) & 0xFFu;
        const uint32_t hi = byte >> 4, lo = byte & 15u;
        float vh, vl;
        if (FMT == kNF4) {
          vh = __uint_as_float(c_nf4_code_bits2[hi]) * s;
          vl = __uint_as_float(c_nf4_code_bits2[lo]) * s;
        } else if (FMT == kFP4) {
          vh = __uint_as_float(c_fp4_code_bits2[hi]) * s;
          vl = __uint_as_float(c_fp4_code_bits2[lo]) * s;
        } else {
          vh = (float)((int)hi - zp) * s;
          vl = (float)((int)lo - zp) * s;
        }
        const uint32_t h16 = __builtin_bit_cast(uint16_t, (_Float16)vh);
        const uint32_t l16 = __builtin_bit_cast(uint16_t, (_Float16)vl);
        o[4 * j + b] = h16 | (l16 << 16);
      }
    }
    uint4* dst = out + c * 4;
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    dst[2] = make_uint4(o[8], o[9], o[10], o[11]);
    dst[3] = make_uint4(o[12], o[13], o[14], o[15]);
  }
}

// Dense GEMV/GEMM over fp16 weights: one wave per (row, 8-wide batch slice); lanes stride over
// 16-byte chunks of the row (8 weights), fp32 accumulation, wave reduction by shuffles.
template <int XT>
__global__ void __launch_bounds__(256) dense_kernel(const uint16_t* __restrict__ x,
                                                     const uint4* __restrict__ w, int64_t n,
                                                     int64_t k, int64_t bsz,
                                                     float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int64_t row = blockIdx.x * 4ll + (threadIdx.x >> 6);
  const int64_t b0 = (int64_t)blockIdx.y * 8;
  if (row >= n) return;
  const int nb = (int)((bsz - b0) < 8 ? (bsz - b0) : 8);
  const int64_t cpr = k >> 3;
  const uint4* wrow = w + row * cpr;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t c = lane; c < cpr; c += 64) {
    const uint4 wp = wrow[c];
    float wf[8];
    const uint32_t wd[4] = {wp.x, wp.y, wp.z, wp.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wf[2 * j] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd[j] & 0xFFFFu));
      wf[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(wd[j] >> 16));
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (b < nb) {
        const uint4 xp = reinterpret_cast<const uint4*>(x + (b0 + b) * k)[c];
        const uint32_t xd[4] = {xp.x, xp.y, xp.z, xp.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float xl, xh;
          if (XT == kF16) {
            xl = (float)__builtin_bit_cast(_Float16, (uint16_t)(xd[j] & 0xFFFFu));
            xh = (float)__builtin_bit_cast(_Float16, (uint16_t)(xd[j] >> 16));
          } else {
            xl = __uint_as_float(xd[j] << 16);
            xh = __uint_as_float(xd[j] & 0xFFFF0000u);
          }
          acc[b] = __builtin_fmaf(wf[2 * j], xl, acc[b]);
          acc[b] = __builtin_fmaf(wf[2 * j + 1], xh, acc[b]);
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    float v = acc[b];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0 && b < nb) y[(b0 + b) * n + row] = v;
  }
}

}  // namespace

hipError_t launch_dequant_f16(int fmt, const uint8_t* packed, const void* scales, int64_t n,
                              int64_t k, uint16_t* w_hat, hipStream_t s) {
  const int cpr = (int)(k / 32);
  const int64_t chunks = n * cpr;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (fmt_weight(fmt) == kFP4) {
    hipLaunchKernelGGL(dequant_kernel<kFP4>, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(packed), scales, chunks, cpr, k,
                       reinterpret_cast<uint4*>(w_hat));
  } else if (fmt_weight(fmt) == kNF4) {
    hipLaunchKernelGGL(dequant_kernel<kNF4>, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(packed), scales, chunks, cpr, k,
                       reinterpret_cast<uint4*>(w_hat));
  } else if (fmt_weight(fmt) == kINT4A) {
    hipLaunchKernelGGL(dequant_kernel<kINT4A>, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(packed), scales, chunks, cpr, k,
                       reinterpret_cast<uint4*>(w_hat));
  } else {
    hipLaunchKernelGGL(dequant_kernel<kINT4>, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(packed), scales, chunks, cpr, k,
                       reinterpret_cast<uint4*>(w_hat));
  }
  return hipGetLastError();
}

hipError_t launch_dense_gemv(int fmt, const uint16_t* x, const uint16_t* w_hat, int64_t n,
                             int64_t k, int64_t b, float* y, hipStream_t s) {
  const dim3 grid((unsigned)((n + 3) / 4), (unsigned)((b + 7) / 8));
  if (fmt_xtype(fmt) == kF16) {
    hipLaunchKernelGGL(dense_kernel<kF16>, grid, dim3(256), 0, s, x,
                       reinterpret_cast<const uint4*>(w_hat), n, k, b, y);
  } else {
    hipLaunchKernelGGL(dense_kernel<kBF16>, grid, dim3(256), 0, s, x,
                       reinterpret_cast<const uint4*>(w_hat), n, k, b, y);
  }
  return hipGetLastError();
}

}  // namespace w4
