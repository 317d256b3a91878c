// 2:4 structured-sparse GEMV: y[b, n] = sum over groups g of four weights of
// v0 x[b, 4g + i0] + v1 x[b, 4g + i1], where (v0, v1) are the row's two kept 16-bit values of the
// group and (i0, i1) their positions (Do Quantization and Sparsity make LLM Inference Faster?,
// "Custom CUDA 2:4 GEMV"): the removed weights are never rebuilt, and the stored bytes are 56.25%
// of dense fp16 ("Library 2:4 sparsity").
//
// Storage per row: K/2 values (fp16 or bf16, the activation's type), two per group; K/8 bytes of
// 4-bit codes, group g in byte g/2 (even groups in the low nibble), code = i0 | i1 << 2.
//
// GEMV layout: a team of T lanes (16, 32 or 64) owns one row; lane t of a team streams the 32-weight
// chunks t, t + T, ... of the row: 32 bytes of values (two 16-byte range-checked loads) and 4
// bytes of codes per chunk.  The lane holds the activations of its chunks in registers for the
// whole launch and walks the workgroup's row blocks with the next block's loads in flight.  Per
// group one v_perm_b32 gathers the activation pair (x[i0], x[i1]) from the group's four
// activations, whose selector is built from the 4-bit code, and one v_dot2 multiplies it with the
// kept pair into fp32.  Team sums by DPP and cross-row shuffles; lane 0 of the team stores.
// A lane holds BT activation rows (1, 2, 4 or 8, as its registers allow for the row length) and
// multiplies each loaded weight group with all of them; slice blockIdx.y takes activation rows
// [BT y, BT y + BT), so only batches larger than BT stream the weights again (the page's kernel
// is batch 1).  Up to four matrices that read the same activations run in one launch,
// their row blocks numbered one after another.
//
// Compression: one thread per two groups (eight weights) keeps the two largest magnitudes of each
// group (ties to the lower position), rounds them to the 16-bit type (nearest even) and writes
// the pair of codes as one byte.
#include "w4_common.h"

namespace w4 {

// Set to non-zero by the compression kernel when it meets a NaN or Inf weight.
__device__ int g_w4_s24_nonfinite;

namespace {

typedef _Float16 s24_half2 __attribute__((ext_vector_type(2)));
typedef __bf16 s24_bf162 __attribute__((ext_vector_type(2)));

constexpr int kS24Threads = 256;
constexpr int kS24MaxItm = 8;

__device__ inline uint32_t to16_bits(float f, int xt) {
  if (xt == kF16) return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // bf16, nearest even (finite inputs)
}

// Positions of the two largest magnitudes of a[0..3], lower position first on ties; returned in
// ascending order.
__device__ inline void keep2(const float (&a)[4], int& p0, int& p1) {
  int rank[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int beaten = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j == i) continue;
      const float ai = fabsf(a[i]), aj = fabsf(a[j]);
      beaten += (aj > ai || (aj == ai && j < i)) ? 1 : 0;
    }
    rank[i] = beaten;
  }
  p0 = -1;
  p1 = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (rank[i] < 2) {
      if (p0 < 0) p0 = i; else p1 = i;
    }
  }
}

__global__ void __launch_bounds__(256) s24_compress_kernel(const float* __restrict__ w, int64_t pairs,
                                                            int xt, uint32_t* __restrict__ values,
                                                            uint8_t* __restrict__ meta) {
  // pair p of groups = weights [8p, 8p + 8) of the flattened [N, K] (K % 32 == 0: no pair
  // crosses a row)
  const int64_t p = blockIdx.x * 256ll + threadIdx.x;
  if (p >= pairs) return;
  const float4 a = reinterpret_cast<const float4*>(w)[2 * p];
  const float4 b = reinterpret_cast<const float4*>(w)[2 * p + 1];
  const float g0[4] = {a.x, a.y, a.z, a.w}, g1[4] = {b.x, b.y, b.z, b.w};
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) bad |= !isfinite(g0[i]) || !isfinite(g1[i]);
  if (bad) g_w4_s24_nonfinite = 1;
  int p0, p1, q0, q1;
  keep2(g0, p0, p1);
  keep2(g1, q0, q1);
  float k0 = g0[0], k1 = g0[1], k2 = g1[0], k3 = g1[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    k0 = i == p0 ? g0[i] : k0;
    k1 = i == p1 ? g0[i] : k1;
    k2 = i == q0 ? g1[i] : k2;
    k3 = i == q1 ? g1[i] : k3;
  }
  values[2 * p] = to16_bits(k0, xt) | (to16_bits(k1, xt) << 16);
  values[2 * p + 1] = to16_bits(k2, xt) | (to16_bits(k3, xt) << 16);
  meta[p] = (uint8_t)((uint32_t)(p0 | (p1 << 2)) | ((uint32_t)(q0 | (q1 << 2)) << 4));
}

template <int CTRL>
__device__ inline float s24_dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}

__device__ inline float s24_team_sum(float v, int team) {
  v += s24_dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += s24_dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += s24_dpp<0x141>(v);  // row_half_mirror
  v += s24_dpp<0x140>(v);  // row_mirror: the 16 lanes of a row hold the row sum
  if (team >= 32) v += __shfl_xor(v, 16);
  if (team >= 64) v += __shfl_xor(v, 32);
  return v;
}

// One matrix of a launch; the members of a grouped launch share x and K, and their row blocks
// are numbered one after another (member g owns row blocks [rb0_g, rb0_g + its row blocks)).
struct S24Member {
  const uint8_t* values;  // [N_g, K] bytes (K/2 16-bit values per row)
  const uint8_t* meta;    // [N_g, K/8]
  float* y;               // [B, N_g]
  int64_t n;
  int64_t rb0;
};

struct S24Args {
  S24Member m[kMaxGroup];
  const uint16_t* x;      // [B, K]
  int64_t k;
  int64_t b;              // activation rows; slice blockIdx.y takes rows [BT y, BT y + BT)
  int64_t nrb;            // row blocks of all members
  int groups;
  int team;
};

template <int XT, int ITM, int BT, bool GROUPED>
__global__ void __launch_bounds__(kS24Threads) s24_gemv_kernel(S24Args a) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int team = a.team;
  const int tshift = __builtin_ctz((unsigned)team);
  const int tl = tid & (team - 1);
  const int team_id = tid >> tshift;
  const int rows_per_wg = kS24Threads >> tshift;
  const int64_t k = a.k;
  const int cpr = (int)(k >> 5);  // 32-weight chunks per row
  const uint32_t vpitch = (uint32_t)k, mpitch = (uint32_t)(k >> 3);
  const int64_t nrb = a.nrb;
  const int64_t b0 = (int64_t)blockIdx.y * BT;                  // this slice's first activation row
  const int64_t nb = a.b - b0 < BT ? a.b - b0 : BT;             // its rows (1..BT)
  // The member owning row block rb (uniform), by selects over the fixed member slots.
  auto member = [&](int64_t rb) {
    S24Member r = a.m[0];
    if constexpr (GROUPED) {
#pragma unroll
      for (int g = 1; g < kMaxGroup; ++g) {
        if (g < a.groups && rb >= a.m[g].rb0) r = a.m[g];
      }
    }
    return r;
  };

  // this lane's activations: chunk c = tl + team * i of each of the slice's rows, 32 values =
  // 16 dwords each (rows past B read as zero)
  uint32_t xr[ITM][BT][16];
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x + b0 * k, (uint32_t)(nb * k * 2));
#pragma unroll
  for (int i = 0; i < ITM; ++i) {
    const int c = tl + team * i;
#pragma unroll
    for (int r = 0; r < BT; ++r) {
      const uint32_t off = offset_or_oob(c < cpr, (uint32_t)(r * k + c * 32) * 2u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = buffer_load16(rx, off + 16u * q);
        xr[i][r][4 * q] = v.x;
        xr[i][r][4 * q + 1] = v.y;
        xr[i][r][4 * q + 2] = v.z;
        xr[i][r][4 * q + 3] = v.w;
      }
    }
  }

  struct Buf {
    uint4 v0[ITM], v1[ITM];
    uint32_t m[ITM];
  };
  // Row block rb's values and codes for this lane, through resources spanning the block's
  // existing rows (rows past N and chunks past the row read as zero).
  auto load = [&](int64_t rb, Buf& d) {
    const S24Member mm = member(rb);
    const int64_t row0 = (rb - mm.rb0) * rows_per_wg;
    const int64_t left = rb < nrb && row0 < mm.n ? mm.n - row0 : 0;
    const uint32_t rows = (uint32_t)(left < rows_per_wg ? left : rows_per_wg);
    const int64_t r0 = left > 0 ? row0 : 0;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(mm.values + r0 * vpitch, rows * vpitch);
    const __amdgpu_buffer_rsrc_t rm = make_rsrc(mm.meta + r0 * mpitch, rows * mpitch);
#pragma unroll
    for (int i = 0; i < ITM; ++i) {
      const int c = tl + team * i;
      const bool have = c < cpr;
      const uint32_t vo = offset_or_oob(have, (uint32_t)team_id * vpitch + (uint32_t)c * 32u);
      d.v0[i] = buffer_load16_stream(rv, vo);
      d.v1[i] = buffer_load16_stream(rv, vo + 16u);
      d.m[i] = buffer_load32(rm, offset_or_oob(have, (uint32_t)team_id * mpitch + (uint32_t)c * 4u));
    }
  };
  auto compute_store = [&](int64_t rb, const Buf& d) {
    float acc[BT];
#pragma unroll
    for (int r = 0; r < BT; ++r) acc[r] = 0.0f;
#pragma unroll
    for (int i = 0; i < ITM; ++i) {
      const uint32_t vals[8] = {d.v0[i].x, d.v0[i].y, d.v0[i].z, d.v0[i].w,
                                d.v1[i].x, d.v1[i].y, d.v1[i].z, d.v1[i].w};
      const uint32_t md = d.m[i];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // code of group j: bits 4j..4j+3; selector bytes (2 i0, 2 i0 + 1, 2 i1, 2 i1 + 1)
        const uint32_t c = (md >> (4 * j)) & 15u;
        const uint32_t spread = ((c << 1) & 6u) | ((c << 15) & 0x60000u);
        const uint32_t sel = spread * 0x101u + 0x01000100u;
#pragma unroll
        for (int r = 0; r < BT; ++r) {
          const uint32_t xp = __builtin_amdgcn_perm(xr[i][r][2 * j + 1], xr[i][r][2 * j], sel);
          if (XT == kF16) {
            acc[r] = __builtin_amdgcn_fdot2(__builtin_bit_cast(s24_half2, vals[j]),
                                            __builtin_bit_cast(s24_half2, xp), acc[r], false);
          } else {
            acc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(s24_bf162, vals[j]),
                                                     __builtin_bit_cast(s24_bf162, xp), acc[r], false);
          }
        }
      }
    }
    const S24Member mm = member(rb);
    const int64_t row = (rb - mm.rb0) * rows_per_wg + team_id;
#pragma unroll
    for (int r = 0; r < BT; ++r) {
      const float v = s24_team_sum(acc[r], team);
      if (tl == 0 && row < mm.n && r < nb) mm.y[(b0 + r) * mm.n + row] = v;
    }
  };

  (void)lane;
  Buf A, Bb;
  int64_t rb = blockIdx.x;
  const int64_t stride = gridDim.x;
  load(rb, A);
  for (; rb < nrb; rb += 2 * stride) {
    load(rb + stride, Bb);  // past the end: rows read as zero, nothing stored
    compute_store(rb, A);
    if (rb + stride >= nrb) break;
    load(rb + 2 * stride, A);
    compute_store(rb + stride, Bb);
  }
}

// Instantiations with ITM x BT <= 8 (activations in at most 128 registers per lane).
template <int XT, int BT, bool GROUPED>
hipError_t launch_itm(int itm, const S24Args& a, dim3 grid, hipStream_t s) {
  switch (itm) {
#define W4_S24(I)                                                                              \
  case I:                                                                                      \
    if constexpr (I * BT <= kS24MaxItm) {                                                      \
      hipLaunchKernelGGL((s24_gemv_kernel<XT, I, BT, GROUPED>), grid, dim3(kS24Threads), 0, s, a); \
      return hipGetLastError();                                                                \
    }                                                                                          \
    break;
    W4_S24(1) W4_S24(2) W4_S24(3) W4_S24(4) W4_S24(5) W4_S24(6) W4_S24(7) W4_S24(8)
#undef W4_S24
  }
  return hipErrorInvalidValue;
}

template <int XT, bool GROUPED>
hipError_t launch_bt(int bt, int itm, const S24Args& a, dim3 grid, hipStream_t s) {
  switch (bt) {
    case 1: return launch_itm<XT, 1, GROUPED>(itm, a, grid, s);
    case 2: return launch_itm<XT, 2, GROUPED>(itm, a, grid, s);
    case 4: return launch_itm<XT, 4, GROUPED>(itm, a, grid, s);
    case 8: return launch_itm<XT, 8, GROUPED>(itm, a, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Team size and chunks per lane for a row of K weights when a lane holds `bt` activation rows:
// the team (16, 32, 64 lanes) whose chunk slots (team x chunks per lane, at most 8 / bt per lane)
// waste the fewest, the smaller team on ties.  Returns false when K needs more slots.
bool sparse24_plan_bt(int64_t k, int bt, int* team, int* itm) {
  const int64_t cpr = k / 32;
  const int64_t max_itm = kS24MaxItm / bt;
  int best_t = 0, best_i = 0;
  int64_t best_waste = -1;
  for (int t = 16; t <= 64; t *= 2) {
    const int64_t i = (cpr + t - 1) / t;
    if (i > max_itm) continue;
    const int64_t waste = t * i - cpr;
    if (best_waste < 0 || waste < best_waste) {
      best_waste = waste;
      best_t = t;
      best_i = (int)i;
    }
  }
  if (best_waste < 0) return false;
  *team = best_t;
  *itm = best_i;
  return true;
}

bool sparse24_plan(int64_t k, int* team, int* itm) { return sparse24_plan_bt(k, 1, team, itm); }

hipError_t launch_sparse24_gemv(int xt, const uint16_t* x, int groups, const uint8_t* const* values,
                                const uint8_t* const* meta, const int64_t* ns, float* const* y,
                                int64_t k, int64_t b, hipStream_t s) {
  // activation rows per slice: the largest power of two <= B whose registers leave a plan
  int team = 0, itm = 0, bt = 8;
  while (bt > b) bt >>= 1;
  while (bt > 1 && !sparse24_plan_bt(k, bt, &team, &itm)) bt >>= 1;
  if (groups < 1 || groups > kMaxGroup || !sparse24_plan_bt(k, bt, &team, &itm))
    return hipErrorInvalidValue;
  const int64_t rows_per_wg = kS24Threads / team;
  S24Args a{};
  int64_t nrb = 0;
  for (int g = 0; g < groups; ++g) {
    a.m[g] = S24Member{values[g], meta[g], y[g], ns[g], nrb};
    nrb += (ns[g] + rows_per_wg - 1) / rows_per_wg;
  }
  for (int g = groups; g < kMaxGroup; ++g) a.m[g] = a.m[0];
  a.x = x;
  a.k = k;
  a.b = b;
  a.nrb = nrb;
  a.groups = groups;
  a.team = team;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int64_t gx = nrb < cap ? nrb : cap;
  const dim3 grid((unsigned)gx, (unsigned)((b + bt - 1) / bt));
  if (groups > 1)
    return xt == kF16 ? launch_bt<kF16, true>(bt, itm, a, grid, s) : launch_bt<kBF16, true>(bt, itm, a, grid, s);
  return xt == kF16 ? launch_bt<kF16, false>(bt, itm, a, grid, s) : launch_bt<kBF16, false>(bt, itm, a, grid, s);
}

hipError_t launch_sparse24_compress(int xt, const float* w, int64_t n, int64_t k, uint16_t* values,
                                    uint8_t* meta, hipStream_t s) {
  const int64_t pairs = n * (k / 8);
  const int64_t blocks = (pairs + 255) / 256;
  hipLaunchKernelGGL(s24_compress_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, pairs, xt,
                     reinterpret_cast<uint32_t*>(values), meta);
  return hipGetLastError();
}

hipError_t sparse24_error_reset(hipStream_t s) {
  const int zero = 0;
  return hipMemcpyToSymbolAsync(HIP_SYMBOL(g_w4_s24_nonfinite), &zero, sizeof(int), 0,
                                hipMemcpyHostToDevice, s);
}

hipError_t sparse24_error_read(int* flag, hipStream_t s) {
  hipError_t e = hipMemcpyFromSymbolAsync(flag, HIP_SYMBOL(g_w4_s24_nonfinite), sizeof(int), 0,
                                          hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace w4
