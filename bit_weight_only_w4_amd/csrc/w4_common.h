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

// FP4 (E2M1) table, fp32: nibbles 0-7 the magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, 8-15 their
// negatives (bit 3 is the sign), as LLM Compressor 0.14, "Details worth knowing" gives the grid.
#define W4_FP4_CODE_BITS                                                                    \
  {0x00000000u, 0x3f000000u, 0x3f800000u, 0x3fc00000u, 0x40000000u, 0x40400000u, 0x40800000u, \
   0x40c00000u, 0x80000000u, 0xbf000000u, 0xbf800000u, 0xbfc00000u, 0xc0000000u, 0xc0400000u, \
   0xc0800000u, 0xc0c00000u}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 128-bit streaming load marked non-temporal (the data is read once).
__device__ inline uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Buffer-resource loads.  A raw buffer resource (base, byte size) makes the hardware range-check
// every access: a load at an offset past the size returns zero and issues no memory request, so
// prefetches of row blocks that do not exist and lanes with no chunk to read cost nothing and need
// no branch.  Word 3 is the gfx9 raw-buffer configuration (32-bit data, no swizzle).
constexpr uint32_t kOutOfRange = 0x7FFFFFF0u;  // past every resource the kernels build

// `off` for lanes that `have` their element, else an offset past the resource.  The select is
// computed as a value (kept opaque to the optimizer) so that the load after it stays a single,
// unconditional instruction: split into branches it would force a wait for all loads in flight.
__device__ inline uint32_t offset_or_oob(bool have, uint32_t off) {
  uint32_t r = have ? off : kOutOfRange;
  asm volatile("" : "+v"(r));
  return r;
}

// `base` and `bytes` must be uniform over the wave; readfirstlane states that to the compiler,
// which otherwise may not prove it and wraps every load in a loop over distinct resources.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint32_t n = (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                           (short)0, (int)n, 0x00020000);
}

// 16 bytes, non-temporal (streamed once).
__device__ inline uint4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline uint32_t buffer_load32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

__device__ inline uint32_t buffer_load16bit(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

// Weight formats.  NF4 and FP4 share the layout (blocks of 64, fp32 scale) and differ only in the
// 16-entry table; INT4 has groups of 128 with a bf16 scale; asymmetric INT4 (INT4A) has the same
// groups with a 32-bit word per group (bf16 scale in bits 0-15, zero point z in bits 16-19).
// INT4A decodes through INT4's table (codes q - 8), and the kernels subtract (z - 8) * s * sum(x)
// per group: (q - z) s = (q - 8) s - (z - 8) s.
enum Fmt { kNF4 = 0, kINT4 = 1, kFP4 = 2, kINT4A = 3 };
enum XType { kF16 = 0, kBF16 = 1 };

// Formats with groups of 128 along K and a bf16 scale.
__host__ __device__ constexpr bool is_g128(int f) { return f == kINT4 || f == kINT4A; }

inline int fmt_weight(int fmt) {
  return (fmt == W4_NF4_X_F16 || fmt == W4_NF4_X_BF16)       ? kNF4
         : (fmt == W4_FP4_X_F16 || fmt == W4_FP4_X_BF16)     ? kFP4
         : (fmt == W4_INT4A_X_F16 || fmt == W4_INT4A_X_BF16) ? kINT4A
                                                             : kINT4;
}
inline int fmt_xtype(int fmt) {
  return (fmt == W4_NF4_X_F16 || fmt == W4_INT4_X_F16 || fmt == W4_FP4_X_F16 ||
          fmt == W4_INT4A_X_F16)
             ? kF16
             : kBF16;
}
inline int64_t fmt_group(int fmt) { return is_g128(fmt_weight(fmt)) ? 128 : 64; }
inline size_t fmt_scale_bytes(int fmt) { return fmt_weight(fmt) == kINT4 ? 2 : 4; }

// Shape of one fused-GEMV launch (host-chosen; see plan_gemv in w4_api.cpp).
struct GemvPlan {
  int threads;  // threads per workgroup (256 or 512)
  int team;     // lanes that share one output row (16..512, power of two, <= threads)
  int iters;    // 16-byte chunks each lane streams per row (<= the instantiated maximum)
  int splits;   // number of disjoint K ranges (grid.y); 1 = single pass
  int cps;      // chunks per split
  int grid_x;   // workgroups along the row dimension
  int cap;      // largest useful grid_x for this shape class (grid_x = min(row blocks, cap))
};

// Matrices of one launch.  A launch covers 1..kMaxGroup weight matrices ("members") that share
// the activations x and K.  Member g is processed by its own range of workgroups along x,
// [wg0, wg0 + grid), which walk its row blocks grid-stride (a single-member launch: all of x).
constexpr int kMaxGroup = W4_MAX_GROUP;

struct GemvMember {
  const uint8_t* packed;  // [N_g, K/2]
  const void* scales;     // NF4, FP4 float[N_g, K/64] | INT4 uint16[N_g, K/128] | INT4A uint32
  float* out;             // y [B, N_g] (splits == 1) or partials [splits, B, N_g]
  uint32_t n;             // rows N_g
  uint32_t nrb;           // row blocks of this member = ceil(N_g / rows per workgroup)
  uint32_t wg0;           // grouped launches: first workgroup (unused slots: 0xFFFFFFFF)
  uint32_t grid;          // grouped launches: workgroups of this member (<= nrb)
};

// Kernel arguments for launches of up to G members (the single-member kernels take G = 1, which
// keeps their argument block at 64 contiguous bytes: the prologue fetches it with one batch of
// scalar loads; a layout that made the compiler split the fetch into two dependent batches cost
// ~0.2 us per launch).
template <int G>
struct GemvArgsT {
  GemvMember m[G];
  const uint16_t* x;  // [B, K] activations (bits), shared by every member
  int64_t k;
  int cpr;            // 16-byte chunks per row = K / 32
  int cps;            // chunks per split
  int team;
  int iters;
  int small_table;    // 1: the decode table holds 16 copies of each entry (4-byte entries; 8 of
                      // the 8-byte ones), written 4x faster, read with up to 4-way conflicts
};
using GemvArgs = GemvArgsT<kMaxGroup>;

constexpr int kGemvMaxThreads = 512;
constexpr int kMaxGemvBatch = 8;

// Largest per-lane chunk count instantiated for batch b (x is held in registers:
// 16 dwords per chunk per batch row).  Grouped launches (several members) are instantiated up to
// 4 chunks per lane, rows of up to 64 Ki weights at 512 lanes per row.
constexpr int gemv_max_iters(int b, bool grouped) {
  return b == 1 ? (grouped ? 4 : 8) : b == 2 ? 4 : b <= 4 ? 2 : 1;
}

// One fused-GEMV launch over `groups` members (a.m[0 .. groups-1]); groups > 1 selects the grouped
// kernels, launched with grid.z = groups.
hipError_t launch_gemv(int fmt, int b, const GemvArgs& a, int groups, const GemvPlan& p,
                       hipStream_t s);
hipError_t launch_splitk_reduce(const float* partial, float* y, int64_t count, int splits,
                                hipStream_t s);
// Device address of the current device's static split-K scratch (W4_NOALLOC_SCRATCH_BYTES),
// looked up once per device.
hipError_t splitk_scratch(void** ptr);
hipError_t launch_quantize_nf4(const float* w, int64_t n, int64_t k, uint8_t* packed,
                               float* absmax, hipStream_t s);
hipError_t launch_quantize_int4(const float* w, int64_t n, int64_t k, uint8_t* packed,
                                uint16_t* scale, hipStream_t s);
hipError_t launch_quantize_int4_asym(const float* w, int64_t n, int64_t k, uint8_t* packed,
                                     uint32_t* words, hipStream_t s);
hipError_t launch_quantize_fp4(const float* w, int64_t n, int64_t k, uint8_t* packed, float* scale,
                               hipStream_t s);
hipError_t quantize_error_reset(hipStream_t s);
hipError_t quantize_error_read(int* flag, hipStream_t s);
hipError_t launch_dequant_f16(int fmt, const uint8_t* packed, const void* scales, int64_t n,
                              int64_t k, uint16_t* w_hat, hipStream_t s);
hipError_t launch_dense_gemv(int fmt, const uint16_t* x, const uint16_t* w_hat, int64_t n,
                             int64_t k, int64_t b, float* y, hipStream_t s);
// MFMA path.  splits > 1 (one member only): K in `splits` ranges of whole quads (fewer when the
// quads do not fill them), each range's partial sums in ws[split][B][N] (fp32), then the
// fixed-order reduction into y; mfma_splits_used gives the number of ranges (0: no plan).
hipError_t launch_mfma(int fmt, const uint16_t* x, const uint8_t* packed, const void* scales,
                       int64_t n, int64_t k, int64_t b, float* y, hipStream_t s, int splits = 1,
                       float* ws = nullptr);
hipError_t launch_mfma_members(int fmt, const uint16_t* x, int groups, const uint8_t* const* packed,
                               const void* const* scales, const int64_t* ns, float* const* y,
                               int64_t k, int64_t b, hipStream_t s, int splits = 1,
                               float* ws = nullptr);
int mfma_splits_used(int64_t n, int64_t k, int64_t b, int splits);
// Tiled GEMM.  splits > 1: K in up to `splits` ranges of whole 64-weight blocks on grid.y
// (gemm_splits_used gives how many), each range's partial sums in ws[range][M][N] (fp32), then the
// fixed-order reduction into y.
hipError_t launch_gemm(int fmt, const uint16_t* x, const uint8_t* packed, const void* scales,
                       int64_t n, int64_t k, int64_t m, float* y, hipStream_t s, int splits = 1,
                       float* ws = nullptr);
int gemm_splits_used(int64_t k, int splits);
// One tiled launch over `groups` members that share x and K (their tiles one after another);
// splits > 1 only with one member.
hipError_t launch_gemm_members(int fmt, const uint16_t* x, int groups, const uint8_t* const* packed,
                               const void* const* scales, const int64_t* ns, float* const* y,
                               int64_t k, int64_t m, hipStream_t s, int splits = 1,
                               float* ws = nullptr);
// Folded-scale GEMM for fp16 activations (w4_gemm_fold.hip): whether a format can run it, the
// weight rows per tile the automatic choice gives an unsplit launch (0: the block-scale kernel is
// faster), the K ranges (and blocks per range) that `splits` give it, the automatic split count
// of the tiled path on one matrix (0: not this kernel), whether split tiled launches take it, and
// one launch over `groups`
// members that share x and K with tiles of `tile_rows` (128 or 256); with more than one K range
// (one member only) the partial sums go to ws ([ranges, M, N] floats) and are added into y.
bool gemm_fold_format(int fmt);
int gemm_fold_tile_rows(int fmt, const int64_t* ns, int groups, int64_t k, int64_t m);
int gemm_fold_ranges(int fmt, int64_t k, int splits, int64_t* bps);
int gemm_fold_auto_splits(int fmt, int64_t n, int64_t k, int64_t m);
bool gemm_fold_split(int fmt, int groups, const int64_t* ns, int64_t m);
hipError_t launch_gemm_fold(int fmt, const uint16_t* x, int groups, const uint8_t* const* packed,
                            const void* const* scales, const int64_t* ns, float* const* y,
                            int64_t k, int64_t m, int tile_rows, hipStream_t s, int splits = 1,
                            float* ws = nullptr);
hipError_t launch_gptq_block(float* w, int64_t ldw, const float* u, int64_t ldu, const float* scale,
                             const float* zero, int64_t lds, int group, int i1, int qmin, int qmax,
                             int64_t rows, int bc, float* q_hat, int64_t ldq, uint8_t* codes,
                             int64_t ldc, float* err, int64_t lde, hipStream_t s);
hipError_t launch_gptq_lazy(float* w, int64_t ldw, const float* err, int64_t lde, const float* u,
                            int64_t ldu, int64_t rows, int64_t cols, int bc, hipStream_t s);
bool sparse24_plan(int64_t k, int* team, int* itm);
hipError_t launch_sparse24_gemv(int xt, const uint16_t* x, int groups, const uint8_t* const* values,
                                const uint8_t* const* meta, const int64_t* ns, float* const* y,
                                int64_t k, int64_t b, hipStream_t s);
hipError_t launch_sparse24_compress(int xt, const float* w, int64_t n, int64_t k, uint16_t* values,
                                    uint8_t* meta, hipStream_t s);
hipError_t sparse24_error_reset(hipStream_t s);
hipError_t sparse24_error_read(int* flag, hipStream_t s);
hipError_t launch_probe_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

int device_cu_count();

}  // namespace w4
