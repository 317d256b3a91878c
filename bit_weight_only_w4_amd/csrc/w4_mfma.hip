// MFMA path for batches of activations: y[b, n] = sum_k x[b, k] * W_hat[n, k] with the weight tile
// decoded on chip and multiplied on the matrix cores (v_mfma_f32_16x16x32_f16 / _bf16, fp32
// accumulation).  At batch 1 a dense-tile rewrite of the fused GEMV loses to the scalar path (My
// Triton Kernel Ties bitsandbytes, "Why Marlin is still faster"); with 16 or more activation rows
// the weight tile is a real dense contraction and the matrix cores pay off.  This path never
// writes decoded weights to memory (LLM Quantization on RTX 4060, "Fused Kernel: Moving
// Dequantization On-Chip").
//
// Work layout (one workgroup = 4 waves = 64 output rows x up to 128 activation rows):
//   * wave w owns rows [64 * blockIdx.x + 16 w, +16); every wave covers all batch tiles
//     (16 activation rows each) and the whole K, in chunks of one scale block: 64 values for NF4,
//     128 for INT4.
//   * A operand (16 rows x 32 k per MFMA step): lane l = 16 g + m takes row m.  In each chunk the
//     lane loads the bytes [8 g, 8 g + 8) (NF4) or [16 g, 16 g + 16) (INT4) of its row's chunk, and
//     MFMA step s uses the s-th dword of them: 8 weights, decoded to 16-bit pairs through the same
//     byte -> pair LDS table as the GEMV.  Every step therefore stays inside one scale block, so
//     the block scale is applied exactly, in fp32, to a fresh per-block accumulator:
//     acc += scale[row, block] * D_block.  No scale is folded into a 16-bit operand.
//   * B operand (32 k x 16 activation rows): lane l = 16 g + n takes activation row n of the tile
//     and the same 8 k positions as the A lane with the same g (one ds_read_b128 from a padded x
//     chunk in LDS, staged by the whole workgroup).
//   * D (16 x 16 fp32): lane l = 16 g + n holds rows 4 g .. 4 g + 3, column n.
//   * NF4 x bf16 uses the two-term bf16 split of each code (two MFMAs per step); INT4 codes q - 8
//     are exact in both 16-bit types.
#include <algorithm>

#include "w4_common.h"

namespace w4 {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kTableBytes = 65536;
constexpr int kMfmaThreads = 256;  // 4 waves, 16 rows each
constexpr int kRowsPerWg = 64;
constexpr int kMaxTiles = 8;       // up to 128 activation rows per launch

__device__ inline uint32_t f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ inline uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline uint32_t nf4_codes_in_lanes() {
  constexpr uint32_t k[16] = W4_NF4_CODE_BITS;
  uint32_t v = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(k[q]), "i"(q));
  return v;
}

template <int FMT, int XT>
__device__ inline void fill_table(uint32_t* tab) {
  uint32_t v1, v2 = 0;
  if (FMT == kNF4) {
    const float c = __uint_as_float(nf4_codes_in_lanes());
    if (XT == kF16) {
      v1 = f16_bits(c);
    } else {
      v1 = bf16_rne_bits(c);
      v2 = bf16_rne_bits(c - __uint_as_float(v1 << 16));
    }
  } else {
    const float v = (float)((int)(threadIdx.x & 15u) - 8);
    v1 = XT == kF16 ? f16_bits(v) : (__float_as_uint(v) >> 16);
  }
  constexpr bool kSplit = (FMT == kNF4 && XT == kBF16);
  uint4* t4 = reinterpret_cast<uint4*>(tab);
  const int tid = threadIdx.x;
  const uint32_t lo1 = (uint32_t)__shfl((int)v1, (tid >> 4) & 15) << 16;
  const uint32_t lo2 = kSplit ? (uint32_t)__shfl((int)v2, (tid >> 4) & 15) << 16 : 0u;
#pragma unroll 4
  for (int j = 0; j < kTableBytes / 16 / kMfmaThreads; ++j) {
    const int i = tid + kMfmaThreads * j;
    const int hi = __builtin_amdgcn_readfirstlane(i >> 8);
    const uint32_t p1 = (uint32_t)__builtin_amdgcn_readlane((int)v1, hi) | lo1;
    if (kSplit) {
      const uint32_t p2 = (uint32_t)__builtin_amdgcn_readlane((int)v2, hi) | lo2;
      t4[i] = make_uint4(p1, p2, p1, p2);
    } else {
      t4[i] = make_uint4(p1, p1, p1, p1);
    }
  }
}

// One 16x16x32 MFMA on 8-value 16-bit fragments (one uint4 each), fp32 accumulate.
template <int XT>
__device__ inline float4_t mfma(const uint4& a, const uint4& b, float4_t c) {
  if constexpr (XT == kF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a),
                                                   __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf168_t, a),
                                                    __builtin_bit_cast(bf168_t, b), c, 0, 0, 0);
  }
}

template <int FMT>
__device__ inline float load_scale(const void* scales, int64_t row, int64_t k, int64_t chunk) {
  if (FMT == kNF4) {
    return reinterpret_cast<const float*>(scales)[row * (k >> 6) + chunk];
  } else {
    const uint16_t s = reinterpret_cast<const uint16_t*>(scales)[row * (k >> 7) + chunk];
    return __uint_as_float((uint32_t)s << 16);
  }
}

struct MfmaArgs {
  const uint16_t* x;      // [B, K]
  const uint8_t* packed;  // [N, K/2]
  const void* scales;
  float* y;               // [B, N]
  int64_t n, k;
  int b;                  // activation rows in this launch (<= 16 * TILES)
};

// KC = weights per chunk along K (64 NF4 / 128 INT4); STEPS = KC / 32 MFMA steps per chunk.
template <int FMT, int XT, int TILES>
__global__ void __launch_bounds__(kMfmaThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
mfma_kernel(MfmaArgs a) {
  constexpr int KC = FMT == kNF4 ? 64 : 128;
  constexpr int STEPS = KC / 32;
  constexpr int XROW = KC * 2 + 16;  // bytes per activation row in LDS (padded against conflicts)
  constexpr int XROWS = 16 * TILES;
  constexpr bool kSplit = (FMT == kNF4 && XT == kBF16);
  __shared__ __align__(16) uint32_t tab[kTableBytes / 4];
  __shared__ __align__(16) uint8_t xs[2][XROWS * XROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, m = lane & 15;
  const int64_t n = a.n, k = a.k;
  const int64_t nchunks = k / KC;
  const int64_t row0 = (int64_t)blockIdx.x * kRowsPerWg + wave * 16;
  const int64_t my_row = row0 + m < n ? row0 + m : n - 1;  // A-operand row of this lane (clamped)

  // --- staging of one x chunk: XROWS x KC halves = XROWS * KC / 8 16-byte pieces
  constexpr int XPIECES = XROWS * KC / 8;
  constexpr int XPER = (XPIECES + kMfmaThreads - 1) / kMfmaThreads;
  uint4 xreg[XPER];
  auto load_x = [&](int64_t c) {
#pragma unroll
    for (int j = 0; j < XPER; ++j) {
      const int piece = tid + j * kMfmaThreads;
      const int r = piece / (KC / 8), q = piece % (KC / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (piece < XPIECES && r < a.b) {
        v = reinterpret_cast<const uint4*>(a.x + (int64_t)r * k + c * KC)[q];
      }
      xreg[j] = v;
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < XPER; ++j) {
      const int piece = tid + j * kMfmaThreads;
      if (piece < XPIECES) {
        const int r = piece / (KC / 8), q = piece % (KC / 8);
        *reinterpret_cast<uint4*>(&xs[buf][r * XROW + q * 16]) = xreg[j];
      }
    }
  };
  // --- this lane's packed bytes of one chunk (8 for NF4, 16 for INT4) and the 4 scales of the
  // rows it holds in D (rows 4 g .. 4 g + 3 of the wave's 16)
  const uint8_t* wrow = a.packed + my_row * (k >> 1);
  auto load_w = [&](int64_t c) -> uint4 {
    if (FMT == kNF4) {
      const uint2 v = *reinterpret_cast<const uint2*>(wrow + c * (KC / 2) + 8 * g);
      return make_uint4(v.x, v.y, 0, 0);
    } else {
      return load_stream16(wrow + c * (KC / 2) + 16 * g);
    }
  };
  auto load_s = [&](int64_t c, float (&s)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t r = row0 + 4 * g + i;
      r = r < n ? r : n - 1;
      s[i] = load_scale<FMT>(a.scales, r, k, c);
    }
  };

  uint4 wcur = load_w(0);
  float scur[4];
  load_s(0, scur);
  load_x(0);
  fill_table<FMT, XT>(tab);
  store_x(0);
  __syncthreads();

  float4_t acc[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  const uint32_t laneoff = kSplit ? (uint32_t)(lane & 31) * 8u : (uint32_t)lane * 4u;
  const char* tabc = reinterpret_cast<const char*>(tab);

  for (int64_t c = 0; c < nchunks; ++c) {
    const int buf = (int)(c & 1);
    // prefetch the next chunk (clamped on the last one: a cache hit, no branch on the loads)
    const int64_t cn = c + 1 < nchunks ? c + 1 : c;
    const uint4 wnext = load_w(cn);
    float snext[4];
    load_s(cn, snext);
    load_x(cn);

    float4_t d[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) d[t] = float4_t{0.f, 0.f, 0.f, 0.f};
    const uint32_t wd[4] = {wcur.x, wcur.y, wcur.z, wcur.w};
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      // decode 8 weights (4 packed bytes) of row m into the A fragment
      uint4 a1, a2 = make_uint4(0, 0, 0, 0);
      uint32_t p1[4], p2[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint32_t addr =
            __builtin_amdgcn_perm(wd[s], laneoff, 0x0C0C0000u | ((4u + (uint32_t)kb) << 8));
        if (kSplit) {
          const uint2 tv = *reinterpret_cast<const uint2*>(tabc + addr);
          p1[kb] = tv.x;
          p2[kb] = tv.y;
        } else {
          p1[kb] = *reinterpret_cast<const uint32_t*>(tabc + addr);
        }
      }
      a1 = make_uint4(p1[0], p1[1], p1[2], p1[3]);
      if (kSplit) a2 = make_uint4(p2[0], p2[1], p2[2], p2[3]);
      // B fragments: activation row (16 t + m), k positions of this lane group and step
      const int koff = FMT == kNF4 ? (16 * g + 8 * s) : (32 * g + 8 * s);
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const uint4 bv = *reinterpret_cast<const uint4*>(&xs[buf][(16 * t + m) * XROW + koff * 2]);
        d[t] = mfma<XT>(a1, bv, d[t]);
        if (kSplit) d[t] = mfma<XT>(a2, bv, d[t]);
      }
    }
    // apply the block scale of each D row in fp32
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      acc[t][0] = __builtin_fmaf(d[t][0], scur[0], acc[t][0]);
      acc[t][1] = __builtin_fmaf(d[t][1], scur[1], acc[t][1]);
      acc[t][2] = __builtin_fmaf(d[t][2], scur[2], acc[t][2]);
      acc[t][3] = __builtin_fmaf(d[t][3], scur[3], acc[t][3]);
    }
    // xs[buf ^ 1] was last read in the previous chunk, which every wave finished before the
    // barrier below was passed last time; one barrier per chunk publishes the new x chunk.
    store_x(buf ^ 1);
    __syncthreads();
    wcur = wnext;
#pragma unroll
    for (int i = 0; i < 4; ++i) scur[i] = snext[i];
  }

  // --- store: lane (g, m) holds y[16 t + m][row0 + 4 g + i], i = 0..3
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const int b = 16 * t + m;
    if (b < a.b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = row0 + 4 * g + i;
        if (r < n) a.y[(int64_t)b * n + r] = acc[t][i];
      }
    }
  }
}

template <int FMT, int XT>
hipError_t launch_fx(const MfmaArgs& a, int tiles, hipStream_t s) {
  const dim3 grid((unsigned)((a.n + kRowsPerWg - 1) / kRowsPerWg));
  switch (tiles) {
    case 1: hipLaunchKernelGGL((mfma_kernel<FMT, XT, 1>), grid, dim3(kMfmaThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((mfma_kernel<FMT, XT, 2>), grid, dim3(kMfmaThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((mfma_kernel<FMT, XT, 4>), grid, dim3(kMfmaThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((mfma_kernel<FMT, XT, 8>), grid, dim3(kMfmaThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Runs the batch in slices of at most 128 activation rows; each slice re-reads the weights.
hipError_t launch_mfma(int fmt, const uint16_t* x, const uint8_t* packed, const void* scales,
                       int64_t n, int64_t k, int64_t b, float* y, hipStream_t s) {
  const int64_t per = 16 * kMaxTiles;
  for (int64_t b0 = 0; b0 < b; b0 += per) {
    MfmaArgs a;
    a.x = x + b0 * k;
    a.packed = packed;
    a.scales = scales;
    a.y = y + b0 * n;
    a.n = n;
    a.k = k;
    a.b = (int)std::min<int64_t>(per, b - b0);
    const int need = (a.b + 15) / 16;
    const int tiles = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
    hipError_t e;
    switch (fmt) {
      case W4_NF4_X_F16: e = launch_fx<kNF4, kF16>(a, tiles, s); break;
      case W4_NF4_X_BF16: e = launch_fx<kNF4, kBF16>(a, tiles, s); break;
      case W4_INT4_X_F16: e = launch_fx<kINT4, kF16>(a, tiles, s); break;
      case W4_INT4_X_BF16: e = launch_fx<kINT4, kBF16>(a, tiles, s); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace w4
