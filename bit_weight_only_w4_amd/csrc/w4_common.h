// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/w4.h"

namespace w4 {

// NF4 code points, fp32, ascending.  The pages fix 16 unevenly spaced codes for normally
// distributed weights stored as fp32 (LLM Quantization on RTX 4060, "Standard Expectation from
// Quantization" and "Kernel Implementation"); the values are the NormalFloat construction
// (normal quantiles at evenly spaced probabilities, 8 positive, 7 negative and an exact zero,
// normalized to [-1, 1]) rounded to fp32, written here as exact bit patterns.
#define W4_NF4_CODE_BITS                                                                    \
  {0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du, 0xbdba7869u, \
   0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u, 0x3ee1a4b5u, 0x3f1007a9u, \
   0x3f3913b0u, 0x3f800000u}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 128-bit streaming load marked non-temporal (the data is read once).
__device__ inline uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

enum Fmt { kNF4 = 0, kINT4 = 1 };
enum XType { kF16 = 0, kBF16 = 1 };

inline int fmt_weight(int fmt) { return (fmt == W4_NF4_X_F16 || fmt == W4_NF4_X_BF16) ? kNF4 : kINT4; }
inline int fmt_xtype(int fmt) { return (fmt == W4_NF4_X_F16 || fmt == W4_INT4_X_F16) ? kF16 : kBF16; }
inline int64_t fmt_group(int fmt) { return fmt_weight(fmt) == kNF4 ? 64 : 128; }

// Shape of one fused-GEMV launch (host-chosen; see choose_gemv in w4_api.cpp).
struct GemvPlan {
  int threads;  // threads per workgroup (64, 128, 256 or 512)
  int team;     // lanes that share one output row (16..512, power of two, <= threads)
  int iters;    // 16-byte chunks each lane streams per row (<= the instantiated maximum)
  int splits;   // number of disjoint K ranges (grid.y); 1 = single pass
  int cps;      // chunks per split
  int grid_x;   // workgroups along the row dimension
};

struct GemvArgs {
  const uint16_t* x;     // [B, K] activations (bits)
  const uint8_t* packed; // [N, K/2]
  const void* scales;    // NF4 float[N, K/64] | INT4 uint16[N, K/128]
  float* out;            // y [B, N] (splits == 1) or partials [splits, B, N]
  int64_t n;
  int64_t k;
  int cpr;               // 16-byte chunks per row = K / 32
  int cps;               // chunks per split
  int team;
  int iters;
  int nrb;               // row blocks = ceil(N / (threads / team)), computed on the host
};

constexpr int kGemvMaxThreads = 512;
constexpr int kMaxGemvBatch = 8;

// Largest per-lane chunk count instantiated for batch b (x is held in registers:
// 16 dwords per chunk per batch row).
inline int gemv_max_iters(int b) { return b == 1 ? 8 : b == 2 ? 4 : b <= 4 ? 2 : 1; }

hipError_t launch_gemv(int fmt, int b, const GemvArgs& a, const GemvPlan& p, hipStream_t s);
hipError_t launch_splitk_reduce(const float* partial, float* y, int64_t count, int splits,
                                hipStream_t s);
hipError_t launch_quantize_nf4(const float* w, int64_t n, int64_t k, uint8_t* packed,
                               float* absmax, hipStream_t s);
hipError_t launch_quantize_int4(const float* w, int64_t n, int64_t k, uint8_t* packed,
                                uint16_t* scale, hipStream_t s);
hipError_t quantize_error_reset(hipStream_t s);
hipError_t quantize_error_read(int* flag, hipStream_t s);
hipError_t launch_dequant_f16(int fmt, const uint8_t* packed, const void* scales, int64_t n,
                              int64_t k, uint16_t* w_hat, hipStream_t s);
hipError_t launch_dense_gemv(int fmt, const uint16_t* x, const uint16_t* w_hat, int64_t n,
                             int64_t k, int64_t b, float* y, hipStream_t s);
hipError_t launch_mfma(int fmt, const uint16_t* x, const uint8_t* packed, const void* scales,
                       int64_t n, int64_t k, int64_t b, float* y, hipStream_t s);
hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

int device_cu_count();

}  // namespace w4
