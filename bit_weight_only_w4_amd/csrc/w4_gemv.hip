// Fused 4-bit dequantize-and-multiply GEMV for gfx950 (CDNA4), batch 1..8, plus the fixed-order
// split-K reduction.
//
// Operation (LLM Quantization on RTX 4060: Where 4-bit Decode Falls Behind FP16, "Kernel
// Implementation"): y[b, n] = sum_k x[b, k] * code(nibble[n, k]) * scale[n, block(k)], reading each
// packed byte once from HBM, decoding on chip and accumulating in fp32.
//
// Layout of the work:
//   * A "team" of T lanes (16..512) owns one output row.  Lane t of a team streams the 16-byte
//     chunks t, t + T, t + 2T, ... of the row (one global_load_dwordx4 each, consecutive lanes on
//     consecutive chunks, so each load instruction covers 64 x 16 contiguous-per-team bytes).
//     A 16-byte chunk is 32 weights: half an NF4 block or a quarter of an INT4 group, so each
//     chunk needs exactly one scale.
//   * The lane keeps the activations of its chunks in VGPRs for the whole launch and loops over
//     the rows of its workgroup with a one-deep prefetch of the next row's packed bytes.
//   * Decode: a 256-entry table in LDS maps a packed byte to the pair (value of the high nibble,
//     value of the low nibble) in the activation's 16-bit type, so one ds_read_b32 decodes two
//     weights.  The table is replicated 64 times with copy c in bank c; lane L reads copy L, so
//     the lookups of a wave never conflict.  The LDS address (byte value * 256 + lane * 4) is
//     built by one v_perm_b32 per byte.
//   * Multiply: v_dot2_f32_f16 / v_dot2_f32_bf16 of the decoded pair with the activation pair,
//     accumulated in fp32 (products of two 16-bit values are exact in fp32); one fp32 FMA per
//     chunk applies the block scale.  NF4 with bf16 activations splits each code into two bf16
//     terms (hi + lo, 8-byte table entries, 32 copies) because a bf16 code alone is not accurate
//     enough.
//   * Reduction over a team: DPP quad/row permutes within 16 lanes, cross-row shuffles up to 64,
//     and an LDS exchange between the waves of a team wider than a wave.
#include "w4_common.h"

namespace w4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

__constant__ uint32_t c_nf4_bits[16] = W4_NF4_CODE_BITS;

constexpr int kTableBytes = 65536;  // 256 entries x 256 bytes

__device__ inline uint32_t f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ inline uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 16-bit decoded value of nibble q in the activation type XT.
template <int FMT, int XT>
__device__ inline uint32_t decode16(uint32_t q) {
  if (FMT == kNF4) {
    float c = __uint_as_float(c_nf4_bits[q]);
    return f16_bits(c);  // fp16 codes (NF4 x bf16 takes the split path below)
  } else {
    float v = (float)((int)q - 8);  // exact small integer
    return XT == kF16 ? f16_bits(v) : (__float_as_uint(v) >> 16);
  }
}

template <int FMT, int XT>
__device__ inline void fill_table(uint32_t* tab) {
  uint4* t4 = reinterpret_cast<uint4*>(tab);
  for (int i = threadIdx.x; i < kTableBytes / 16; i += blockDim.x) {
    const uint32_t e = (uint32_t)i >> 4;  // 16 uint4 = 256 bytes per entry
    const uint32_t hi = e >> 4, lo = e & 15u;
    uint4 v;
    if (FMT == kNF4 && XT == kBF16) {
      const float ch = __uint_as_float(c_nf4_bits[hi]);
      const float cl = __uint_as_float(c_nf4_bits[lo]);
      const uint32_t h1 = bf16_rne_bits(ch), l1 = bf16_rne_bits(cl);
      const uint32_t h2 = bf16_rne_bits(ch - __uint_as_float(h1 << 16));
      const uint32_t l2 = bf16_rne_bits(cl - __uint_as_float(l1 << 16));
      const uint32_t p1 = h1 | (l1 << 16), p2 = h2 | (l2 << 16);
      v = make_uint4(p1, p2, p1, p2);
    } else {
      const uint32_t p = decode16<FMT, XT>(hi) | (decode16<FMT, XT>(lo) << 16);
      v = make_uint4(p, p, p, p);
    }
    t4[i] = v;
  }
}

template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}

// Sum over the lanes of a team of `team` lanes (team <= 64) inside one wave; every lane of the
// team ends with the total.
__device__ inline float team_sum_wave(float v, int team) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror: all 16 lanes of a row hold the row sum
  if (team >= 32) v += __shfl_xor(v, 16);
  if (team >= 64) v += __shfl_xor(v, 32);
  return v;
}

template <int FMT>
__device__ inline float load_scale(const void* scales, int64_t row, int64_t k, int chunk) {
  if (FMT == kNF4) {
    return reinterpret_cast<const float*>(scales)[row * (k >> 6) + (chunk >> 1)];
  } else {
    const uint16_t s = reinterpret_cast<const uint16_t*>(scales)[row * (k >> 7) + (chunk >> 2)];
    return __uint_as_float((uint32_t)s << 16);
  }
}

template <int FMT, int XT, int B, int ITM>
__global__ void __launch_bounds__(kGemvThreads) gemv_kernel(GemvArgs a) {
  __shared__ __align__(16) uint32_t tab[kTableBytes / 4];
  __shared__ float xwave[kGemvThreads / 64][B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int team = a.team;
  const int tshift = __builtin_ctz((unsigned)team);
  const int tl = tid & (team - 1);
  const int team_id = tid >> tshift;
  const int teams_per_wg = kGemvThreads >> tshift;
  const int c0 = blockIdx.y * a.cps;
  const int nck = min(a.cps, a.cpr - c0);
  const int64_t n = a.n, k = a.k;
  const int64_t nrb = (n + teams_per_wg - 1) / teams_per_wg;

  // --- first row's packed bytes and scales: issued before anything else
  uint4 pk[ITM];
  float sc[ITM];
  int64_t rb = blockIdx.x;
  auto load_row = [&](int64_t rbv, uint4 (&p)[ITM], float (&s)[ITM]) {
    int64_t row = rbv * teams_per_wg + team_id;
    row = row < n ? row : n - 1;
    const uint4* prow = reinterpret_cast<const uint4*>(a.packed + row * (k >> 1));
#pragma unroll
    for (int i = 0; i < ITM; ++i) {
      const int c = tl + (i << tshift);
      if (i < a.iters && c < nck) {
        p[i] = load_stream16(prow + c0 + c);
        s[i] = load_scale<FMT>(a.scales, row, k, c0 + c);
      } else {
        p[i] = make_uint4(0, 0, 0, 0);
        s[i] = 0.0f;
      }
    }
  };
  if (rb < nrb) load_row(rb, pk, sc);

  // --- activations of this lane's chunks, kept in VGPRs (zero for chunks past the range)
  uint32_t xr[ITM][B][16];
#pragma unroll
  for (int i = 0; i < ITM; ++i) {
    const int c = tl + (i << tshift);
    const bool ok = i < a.iters && c < nck;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const uint4* xb = reinterpret_cast<const uint4*>(a.x + b * k) + (int64_t)(c0 + (ok ? c : 0)) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = ok ? xb[q] : make_uint4(0, 0, 0, 0);
        xr[i][b][4 * q + 0] = v.x;
        xr[i][b][4 * q + 1] = v.y;
        xr[i][b][4 * q + 2] = v.z;
        xr[i][b][4 * q + 3] = v.w;
      }
    }
  }

  // --- decode table (overlaps the first loads' latency)
  fill_table<FMT, XT>(tab);
  __syncthreads();

  constexpr bool kSplitCode = (FMT == kNF4 && XT == kBF16);
  const uint32_t laneoff = kSplitCode ? (uint32_t)(lane & 31) * 8u : (uint32_t)lane * 4u;
  const char* tabc = reinterpret_cast<const char*>(tab);
  const int wave = tid >> 6;
  const int waves_per_team = team > 64 ? team >> 6 : 1;

  for (; rb < nrb; rb += gridDim.x) {
    uint4 npk[ITM];
    float nsc[ITM];
    const int64_t nxt = rb + gridDim.x;
    if (nxt < nrb) load_row(nxt, npk, nsc);

    float acc[B];
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = 0.0f;

#pragma unroll
    for (int i = 0; i < ITM; ++i) {
      const int c = tl + (i << tshift);
      if (i < a.iters && c < nck) {
        float d[B];
#pragma unroll
        for (int b = 0; b < B; ++b) d[b] = 0.0f;
        const uint32_t wv[4] = {pk[i].x, pk[i].y, pk[i].z, pk[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            // LDS byte address: lane offset in byte 0, the packed byte in byte 1.
            const uint32_t addr =
                __builtin_amdgcn_perm(wv[j], laneoff, 0x0C0C0000u | ((4u + (uint32_t)kb) << 8));
            const int m = 4 * j + kb;  // byte index in the chunk = activation pair index
            if (kSplitCode) {
              const uint2 t = *reinterpret_cast<const uint2*>(tabc + addr);
#pragma unroll
              for (int b = 0; b < B; ++b) {
                const bf162_t xv = __builtin_bit_cast(bf162_t, xr[i][b][m]);
                d[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, t.x), xv, d[b], false);
                d[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, t.y), xv, d[b], false);
              }
            } else {
              const uint32_t t = *reinterpret_cast<const uint32_t*>(tabc + addr);
#pragma unroll
              for (int b = 0; b < B; ++b) {
                if (XT == kF16) {
                  d[b] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, t),
                                                __builtin_bit_cast(half2_t, xr[i][b][m]), d[b], false);
                } else {
                  d[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, t),
                                                         __builtin_bit_cast(bf162_t, xr[i][b][m]), d[b],
                                                         false);
                }
              }
            }
          }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) acc[b] = __builtin_fmaf(d[b], sc[i], acc[b]);
      }
    }

    const int64_t row = rb * teams_per_wg + team_id;
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = team_sum_wave(acc[b], team);
    float* out = a.out + (int64_t)blockIdx.y * B * n;
    if (waves_per_team == 1) {
      if (tl == 0 && row < n) {
#pragma unroll
        for (int b = 0; b < B; ++b) out[b * n + row] = acc[b];
      }
    } else {
      if (lane == 0) {
#pragma unroll
        for (int b = 0; b < B; ++b) xwave[wave][b] = acc[b];
      }
      __syncthreads();
      if (tl == 0 && row < n) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float v = 0.0f;
          for (int w = 0; w < waves_per_team; ++w) v += xwave[wave + w][b];
          out[b * n + row] = v;
        }
      }
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < ITM; ++i) {
      pk[i] = npk[i];
      sc[i] = nsc[i];
    }
  }
}

__global__ void splitk_reduce_kernel(const float* __restrict__ partial, float* __restrict__ y,
                                     int64_t count, int splits) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v = 0.0f;
    for (int s = 0; s < splits; ++s) v += partial[s * count + i];  // fixed order s = 0, 1, ...
    y[i] = v;
  }
}

template <int FMT, int XT, int B, int ITM>
hipError_t launch_one(const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  hipLaunchKernelGGL((gemv_kernel<FMT, XT, B, ITM>), dim3(p.grid_x, p.splits), dim3(kGemvThreads),
                     0, s, a);
  return hipGetLastError();
}

template <int FMT, int XT, int B>
hipError_t launch_b(const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  const int it = p.iters;
  if constexpr (B == 1) {
    switch (it) {
      case 1: return launch_one<FMT, XT, B, 1>(a, p, s);
      case 2: return launch_one<FMT, XT, B, 2>(a, p, s);
      case 3: return launch_one<FMT, XT, B, 3>(a, p, s);
      case 4: return launch_one<FMT, XT, B, 4>(a, p, s);
      case 5: return launch_one<FMT, XT, B, 5>(a, p, s);
      case 6: return launch_one<FMT, XT, B, 6>(a, p, s);
      case 7: return launch_one<FMT, XT, B, 7>(a, p, s);
      case 8: return launch_one<FMT, XT, B, 8>(a, p, s);
    }
  } else if constexpr (B == 2) {
    switch (it) {
      case 1: return launch_one<FMT, XT, B, 1>(a, p, s);
      case 2: return launch_one<FMT, XT, B, 2>(a, p, s);
      case 3: return launch_one<FMT, XT, B, 3>(a, p, s);
      case 4: return launch_one<FMT, XT, B, 4>(a, p, s);
    }
  } else if constexpr (B <= 4) {
    switch (it) {
      case 1: return launch_one<FMT, XT, B, 1>(a, p, s);
      case 2: return launch_one<FMT, XT, B, 2>(a, p, s);
    }
  } else {
    if (it == 1) return launch_one<FMT, XT, B, 1>(a, p, s);
  }
  return hipErrorInvalidValue;
}

template <int FMT, int XT>
hipError_t launch_fx(int b, const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  switch (b) {
    case 1: return launch_b<FMT, XT, 1>(a, p, s);
    case 2: return launch_b<FMT, XT, 2>(a, p, s);
    case 3: return launch_b<FMT, XT, 3>(a, p, s);
    case 4: return launch_b<FMT, XT, 4>(a, p, s);
    case 5: return launch_b<FMT, XT, 5>(a, p, s);
    case 6: return launch_b<FMT, XT, 6>(a, p, s);
    case 7: return launch_b<FMT, XT, 7>(a, p, s);
    case 8: return launch_b<FMT, XT, 8>(a, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemv(int fmt, int b, const GemvArgs& a, const GemvPlan& p, hipStream_t s) {
  switch (fmt) {
    case W4_NF4_X_F16: return launch_fx<kNF4, kF16>(b, a, p, s);
    case W4_NF4_X_BF16: return launch_fx<kNF4, kBF16>(b, a, p, s);
    case W4_INT4_X_F16: return launch_fx<kINT4, kF16>(b, a, p, s);
    case W4_INT4_X_BF16: return launch_fx<kINT4, kBF16>(b, a, p, s);
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
