// MFMA path for batches of activations: y[b, n] = sum_k x[b, k] * W_hat[n, k] with the weight tile
// decoded on chip and multiplied on the matrix cores (v_mfma_f32_16x16x32_f16 / _bf16, fp32
// accumulation).  At batch 1 a dense-tile rewrite of the fused GEMV loses to the scalar path (My
// Triton Kernel Ties bitsandbytes, "Why Marlin is still faster"); once several activation rows
// share each decoded weight, the per-weight multiply work of the scalar path grows with the batch
// while one matrix-core step covers 16 activation rows.  Decoded weights never go to memory (LLM
// Quantization on RTX 4060, "Fused Kernel: Moving Dequantization On-Chip").
//
// Work layout.  A workgroup has 8 waves = RW row groups x KW K groups (RW * KW = 8).  Row group rg
// owns 16 output rows; K group kg owns a contiguous range of K: quads kg * qpk .. kg * qpk + qpk - 1,
// a quad being 256 weights (4 NF4 blocks or 2 INT4 groups).  Every wave covers all T batch tiles
// (16 activation rows each).
//   * A operand (16 rows x 32 k per MFMA step): lane l = 16 g + m takes row m.  In a scale block of
//     KC weights (64 NF4 / 128 INT4) each lane group holds KC/8 bytes of its row's block (which
//     bytes: see Quad; K is permuted freely inside a block, x follows the same order); MFMA step s
//     uses their s-th dword, 8 weights decoded to 16-bit pairs through the same byte -> pair LDS
//     table as the GEMV.  Each step lies inside one scale block, so the block scale is applied
//     exactly, in fp32, to a fresh per-block result: acc += scale[row] * D_block.
//   * Packed bytes arrive in 16-byte loads per lane (a wave reads 64 contiguous bytes of each of
//     its 16 rows per load); for NF4 a lane-half swap then gives each lane group its 8 bytes of
//     each 32-byte block.
//   * Weights and scales stream from HBM through range-checked buffer loads into registers, two
//     quads ahead of the quad being multiplied; the two register sets alternate by unrolling, so
//     a refill never waits on its own previous load.
//   * B operand (32 k x 16 activation rows): lane l = 16 g + n takes activation row n of the tile
//     and the same 8 k positions as the A lane with the same g: one ds_read_b128 from an x window
//     in LDS.  The window holds, for every batch row, qpp quads of each K group; it is reloaded
//     once per phase of qpp quads, which the host sizes to fill the LDS the table leaves.
//   * D (16 x 16 fp32): lane l = 16 g + n holds rows 4 g .. 4 g + 3, column n.
//   * K groups end by adding their results in LDS in the fixed order kg = 0, 1, ..., KW - 1, so the
//     output is bitwise reproducible.
//   * NF4 x bf16 uses the two-term bf16 split of each code (two MFMAs per step); INT4 codes q - 8
//     are exact in both 16-bit types.
#include <algorithm>

#include "w4_common.h"

namespace w4 {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTableBytes = 32768;   // 256 entries x 128 bytes
constexpr int kThreads = 512;        // 8 waves
constexpr int kXBytes = 128 * 1024;  // x window; the table takes the other 32 KiB of the 160 KiB
constexpr int kQuad = 256;          // weights per quad
constexpr int kMaxTiles = 8;        // up to 128 activation rows per launch

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

// The byte -> decoded pair table, as in the GEMV kernel but with 32 copies of each 4-byte entry
// (16 of each 8-byte NF4 x bf16 entry): 128 bytes per entry, lane L reading copy L % 32 (L % 16).
// Half the GEMV's LDS, which leaves room for a larger x window.
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
  // 16-byte slot i belongs to entry i >> 3: high nibble i >> 7 (uniform over a wave), low nibble
  // (i >> 3) & 15 (the same for every slot of a thread).
  const uint32_t lo1 = (uint32_t)__shfl((int)v1, (tid >> 3) & 15) << 16;
  const uint32_t lo2 = kSplit ? (uint32_t)__shfl((int)v2, (tid >> 3) & 15) << 16 : 0u;
#pragma unroll 4
  for (int j = 0; j < kTableBytes / 16 / kThreads; ++j) {
    const int i = tid + kThreads * j;
    const int hi = __builtin_amdgcn_readfirstlane(i >> 7);
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

struct MfmaArgs {
  const uint16_t* x;      // [B, K]
  const uint8_t* packed;  // [N, K/2]
  const void* scales;     // NF4 float[N, K/64] | INT4 uint16[N, K/128]
  float* y;               // [B, N]
  int64_t n, k;
  int b;       // activation rows in all; slice blockIdx.y takes rows [16 T y, 16 T (y + 1))
  int qpk;     // quads per K group
  int qpp;     // quads per K group in one x window (one phase)
  int xrow;    // bytes per activation row of the x window: KW * qpp * 512 + 16
  int tiles;   // row tiles (16 * RW rows each) in all
};

// One quad in this lane's registers: 32 packed bytes of its A row (two 16-byte loads), and the
// scale of one D row per block: lane (g, m) holds row 4 g + (m & 3), and lane (g, n) gets the
// scales of its rows 4 g + i from lanes (g, i) by a DPP row broadcast.
//   INT4 (2 blocks of 64 bytes): load c holds bytes [16 g, 16 g + 16) of block c.
//   NF4 (4 blocks of 32 bytes): load h holds bytes [16 g, 16 g + 16) of the 64 bytes of blocks
//   2 h, 2 h + 1, so lane groups 0, 1 hold block 2 h and groups 2, 3 block 2 h + 1.  Two
//   v_permlane32_swap give every lane 8 bytes of each block: lane group L then holds the bytes
//   [16 g0, 16 g0 + 8) of both blocks' lane-group-(L & 1) halves, g0 = L & 1, offset by 8 bytes
//   for L >= 2, i.e. the 16 weights from 32 (L & 1) + 16 (L >> 1) of each block.
template <int FMT>
struct Quad {
  static constexpr int QC = FMT == kNF4 ? 4 : 2;  // scale blocks per quad
  uint32_t w[2][4];
  uint32_t s[QC];  // fp32 bits (INT4: bf16 bits shifted to the high half)
};

// Lane i of each row of 16 lanes, broadcast to the row.
template <int I>
__device__ inline float row_bcast(uint32_t v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + I, 0xF, 0xF, false));
}

template <int FMT, int XT, int T, int KW>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
mfma_kernel(MfmaArgs a) {
  constexpr int RW = 8 / KW;
  constexpr int KC = FMT == kNF4 ? 64 : 128;  // weights per scale block
  constexpr int QC = kQuad / KC;              // blocks per quad
  constexpr int STEPS = KC / 32;              // MFMA steps per block
  constexpr int SB = FMT == kNF4 ? 4 : 2;     // bytes per scale
  constexpr bool kSplit = (FMT == kNF4 && XT == kBF16);
  __shared__ __align__(16) uint32_t tab[kTableBytes / 4];
  __shared__ __align__(16) uint8_t xs[kXBytes];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = wave % RW, kg = wave / RW;
  const int g = lane >> 4, m = lane & 15;
  const int64_t n = a.n, k = a.k;
  const int64_t nblocks = k / KC;
  const uint32_t pitch = (uint32_t)(k >> 1);
  const uint32_t spitch = (uint32_t)(nblocks * SB);
  // This workgroup's batch slice: activation rows [16 T y, 16 T y + bsl).
  const int64_t b0 = (int64_t)blockIdx.y * 16 * T;
  const int bsl = (int)min((int64_t)16 * T, (int64_t)a.b - b0);
  const uint16_t* xsl = a.x + b0 * k;
  float* ysl = a.y + b0 * n;
  const __amdgpu_buffer_rsrc_t rx_ = make_rsrc(xsl, (uint32_t)(bsl * k * 2));

  // The workgroup's row tiles: blockIdx.x, blockIdx.x + gridDim.x, ...  A workgroup runs several
  // tiles (a persistent grid) only when the whole of x fits one window and KW == 1; otherwise the
  // grid has one workgroup per tile.
  const int ntiles = ((int)a.tiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int nq = a.qpk;               // quads per tile and wave
  const int64_t len = (int64_t)ntiles * nq;  // this wave's stream of (tile, quad) positions

  // Per-lane byte offsets inside a row tile: the A bytes of row m / lane group g, and the scale
  // row 4 g + (m & 3) (see Quad).
  const uint32_t wlane = (uint32_t)m * pitch + (uint32_t)(g * 16);
  const uint32_t slane = (uint32_t)(4 * g + (m & 3)) * spitch;

  // A cursor over this wave's stream of (tile ti, quad q) positions, with the buffer resources of
  // tile ti's 16 rows (rows past N, and tiles past the stream, read as zero).
  struct Cursor {
    int ti, q;
    __amdgpu_buffer_rsrc_t rw, rs;
  };
  auto set_tile = [&](Cursor& c) __attribute__((always_inline)) {
    const int64_t row_base = ((int64_t)(blockIdx.x + (int64_t)c.ti * gridDim.x) * RW + rg) * 16;
    const int64_t rows_left = c.ti < ntiles ? n - row_base : 0;
    const uint32_t rows = rows_left <= 0 ? 0u : rows_left >= 16 ? 16u : (uint32_t)rows_left;
    c.rw = make_rsrc(a.packed + row_base * pitch, rows * pitch);
    c.rs = make_rsrc(reinterpret_cast<const char*>(a.scales) + row_base * spitch, rows * spitch);
  };
  // (Branch-free: the counters stay scalar values the compiler can keep in registers.)
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    const bool wrap = c.q + 1 == nq;
    c.q = wrap ? 0 : c.q + 1;
    c.ti += wrap ? 1 : 0;
    set_tile(c);
  };
  // The quad at the cursor: blocks qb .. qb + QC - 1 of the K group, qb = (kg * qpk + q) * QC.
  // Blocks past K read as zero (their weights and scales), which adds nothing.  Each lane's 16
  // bytes lie inside one block.
  const int lblk = FMT == kNF4 ? (g >> 1) : 0;  // block of this lane's bytes within a load
  auto load_quad = [&](const Cursor& cur, Quad<FMT>& d) __attribute__((always_inline)) {
    const uint32_t qb = (uint32_t)((kg * a.qpk + cur.q) * QC);
    const uint32_t wbase = wlane + qb * (KC / 2);
    const uint32_t sbase = slane + qb * SB;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int blk = FMT == kNF4 ? 2 * h + lblk : h;
      const bool have = (int64_t)qb + blk < nblocks;
      const uint4 v = buffer_load16_stream(cur.rw, offset_or_oob(have, wbase + 64u * h));
      d.w[h][0] = v.x;
      d.w[h][1] = v.y;
      d.w[h][2] = v.z;
      d.w[h][3] = v.w;
    }
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      const bool have = (int64_t)qb + c < nblocks;
      const uint32_t so = offset_or_oob(have, sbase) + (uint32_t)(c * SB);
      d.s[c] = FMT == kNF4 ? buffer_load32(cur.rs, so) : buffer_load16bit(cur.rs, so) << 16;
    }
  };

  // x window of phase p: for every batch row r < 16 T and K group kk, its quads
  // kk * qpk + p * qpp .. + qpp - 1; rows past B and k past K are zero.  The window is copied
  // straight from global memory into LDS (buffer loads with the LDS destination): 16-byte slot
  // s = tid + 512 j of the window area receives lane (s % 64)'s load, so slot s holds piece
  // col = s % (rowp + 1) of row r = s / (rowp + 1), the last piece of a row being the padding.
  const int xrow = a.xrow;
  const int seg = a.qpp * (kQuad / 8);  // 16-byte pieces of one K group's segment of a row
  const int rowp = KW * seg;            // data pieces per window row (<= 480)
  const int slots = 16 * T * (rowp + 1);
  const int nphase = (nq + a.qpp - 1) / a.qpp;
  // Integer quotients through float reciprocals: s < 8192 and, after the + 0.5 offset, s / (rowp
  // + 1) and col / seg stay at least 1 / 962 away from an integer, far above the error of the fp32
  // reciprocal and product.
  const float inv_row = 1.0f / (float)(rowp + 1);
  const float inv_seg = 1.0f / (float)seg;
  constexpr int kXPer = kXBytes / 16 / kThreads;  // 16 slots per thread cover the whole area
  auto load_x = [&](int p) __attribute__((always_inline)) {
    const int64_t kbase = (int64_t)p * a.qpp * kQuad;
    // Recomputed at each window rather than kept live across the main loop (registers).
    int t0 = tid;
    asm volatile("" : "+v"(t0));
#pragma unroll
    for (int j = 0; j < kXPer; ++j) {
      const int sl = t0 + j * kThreads;
      const int r = (int)(((float)sl + 0.5f) * inv_row);
      const int col = sl - r * (rowp + 1);
      const int kk = (int)(((float)col + 0.5f) * inv_seg);
      const int pc = col - kk * seg;
      const int64_t kpos = (int64_t)kk * a.qpk * kQuad + kbase + (int64_t)pc * 8;
      const bool have = sl < slots && col < rowp && r < bsl && kpos < k;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx_, (__attribute__((address_space(3))) void*)(xs + (j * kThreads + wave * 64) * 16), 16,
          (int)offset_or_oob(have, (uint32_t)((r * k + kpos) * 2)), 0, 0, 0);
    }
  };

  // The load cursor runs R positions ahead of the compute cursor (R register sets; two for 8
  // batch tiles, whose accumulators leave no room for four).
  constexpr int R = T == 8 ? 2 : 4;
  Cursor ld;
  ld.ti = 0;
  ld.q = 0;
  set_tile(ld);
  Quad<FMT> P0, P1, P2, P3;
  load_quad(ld, P0);
  advance(ld);
  load_quad(ld, P1);
  advance(ld);
  if constexpr (R == 4) {
    load_quad(ld, P2);
    advance(ld);
    load_quad(ld, P3);
    advance(ld);
  }
  load_x(0);
  fill_table<FMT, XT>(tab);
  __syncthreads();

  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Twice this lane's byte offset in a table entry (see the lookup below).
  const uint32_t laneoff = kSplit ? (uint32_t)(lane & 15) * 16u : (uint32_t)(lane & 31) * 8u;
  const char* tabc = reinterpret_cast<const char*>(tab);
  const uint8_t* xw = xs + kg * (seg * 16) + m * xrow;  // this lane's B row (tile 0), K group kg

  // k offset (in the block) of the first of this lane's weights for MFMA step 0 (see Quad).
  const int klane = FMT == kNF4 ? 32 * (g & 1) + 16 * (g >> 1) : 32 * g;

  // Multiply the quad held in d; wq = its index inside the current x window.
  auto compute = [&](int wq, const Quad<FMT>& d) __attribute__((always_inline)) {
    // this lane's 2 (NF4) or 4 (INT4) dwords of packed bytes per block
    uint32_t wb[QC][STEPS];
    if constexpr (FMT == kNF4) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto s0 = __builtin_amdgcn_permlane32_swap(d.w[h][0], d.w[h][2], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(d.w[h][1], d.w[h][3], false, false);
        wb[2 * h][0] = s0[0];
        wb[2 * h][1] = s1[0];
        wb[2 * h + 1][0] = s0[1];
        wb[2 * h + 1][1] = s1[1];
      }
    } else {
#pragma unroll
      for (int c = 0; c < QC; ++c) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s) wb[c][s] = d.w[c][s];
      }
    }
    const uint8_t* xq = xw + (wq * kQuad + klane) * 2;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      float4_t dd[T];
#pragma unroll
      for (int t = 0; t < T; ++t) dd[t] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < STEPS; ++s) {
        uint32_t p1[4], p2[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          // LDS byte address = byte * 128 + lane offset: the perm builds byte * 256 + 2 * lane
          // offset (the packed byte into byte 1), halved by the shift.
          const uint32_t addr =
              __builtin_amdgcn_perm(wb[c][s], laneoff, 0x0C0C0000u | ((4u + (uint32_t)kb) << 8)) >> 1;
          if (kSplit) {
            const uint2 tv = *reinterpret_cast<const uint2*>(tabc + addr);
            p1[kb] = tv.x;
            p2[kb] = tv.y;
          } else {
            p1[kb] = *reinterpret_cast<const uint32_t*>(tabc + addr);
          }
        }
        const uint4 a1 = make_uint4(p1[0], p1[1], p1[2], p1[3]);
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const uint4 bv =
              *reinterpret_cast<const uint4*>(xq + 16 * t * xrow + (c * KC + s * 8) * 2);
          dd[t] = mfma<XT>(a1, bv, dd[t]);
          if (kSplit) dd[t] = mfma<XT>(make_uint4(p2[0], p2[1], p2[2], p2[3]), bv, dd[t]);
        }
        // With 8 tiles, keep each step's B fragments from being fetched ahead of the previous
        // step (they would not fit the registers left by the accumulators).
        if constexpr (T == 8) __builtin_amdgcn_sched_barrier(0);
      }
      const float sc[4] = {row_bcast<0>(d.s[c]), row_bcast<1>(d.s[c]), row_bcast<2>(d.s[c]),
                           row_bcast<3>(d.s[c])};
#pragma unroll
      for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(dd[t][i], sc[i], acc[t][i]);
      }
    }
  };

  // y rows of tile ti: after its last quad, K groups add up (KW > 1, one tile per workgroup) and
  // kg == 0 stores; lane (g, m) holds y[16 t + m][row_d + i], i = 0..3.
  auto finish_tile = [&](int ti) __attribute__((always_inline)) {
    const int64_t row_d = ((int64_t)(blockIdx.x + (int64_t)ti * gridDim.x) * RW + rg) * 16 + 4 * g;
    if constexpr (KW > 1) {
      float4_t* red = reinterpret_cast<float4_t*>(xs);  // [KW - 1][RW][T][64 lanes]
      __syncthreads();
      if (kg > 0) {
#pragma unroll
        for (int t = 0; t < T; ++t) red[(((kg - 1) * RW + rg) * T + t) * 64 + lane] = acc[t];
      }
      __syncthreads();
      if (kg == 0) {
        for (int j = 1; j < KW; ++j) {
#pragma unroll
          for (int t = 0; t < T; ++t) {
            const float4_t v = red[(((j - 1) * RW + rg) * T + t) * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] += v[i];
          }
        }
      }
    }
    if (kg == 0) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int b = 16 * t + m;
        if (b < bsl) {
          float* yr = ysl + (int64_t)b * n;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (row_d + i < n) yr[row_d + i] = acc[t][i];
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  };

  // One stream position with the quad in d: a new x window at every multiple of qpp quads (only
  // when the tile needs several windows, i.e. one tile per workgroup), the multiply, the refill of
  // d R positions ahead, and the end of the tile after its last quad.
  int ct = 0, cq = 0;
  auto step = [&](Quad<FMT>& d) __attribute__((always_inline)) {
    if (nphase > 1 && cq > 0 && cq % a.qpp == 0) {
      __syncthreads();  // every wave is done with the old window
      load_x(cq / a.qpp);
      __syncthreads();
    }
    compute(nphase > 1 ? cq % a.qpp : cq, d);
    load_quad(ld, d);
    advance(ld);
    const bool last = cq == nq - 1;
    if (last) finish_tile(ct);
    ct += last ? 1 : 0;
    cq = last ? 0 : cq + 1;
  };

  // Main loop: R positions per trip, the register sets rotating without copies; the last
  // positions are already loaded when it ends.
  int64_t j = 0;
  if constexpr (R == 4) {
    for (; j + 4 <= len; j += 4) {
      step(P0);
      step(P1);
      step(P2);
      step(P3);
    }
    if (j < len) step(P0);
    if (j + 1 < len) step(P1);
    if (j + 2 < len) step(P2);
  } else {
    for (; j + 2 <= len; j += 2) {
      step(P0);
      step(P1);
    }
    if (j < len) step(P0);
  }
}

// K groups the x window allows for T batch tiles (plan_mfma never asks for more): 8 / 4 / 2 / 1.
constexpr int max_kw(int t) { return t == 1 ? 8 : t == 2 ? 4 : t == 4 ? 2 : 1; }

template <int FMT, int XT, int T, int KW>
hipError_t launch_kw(const MfmaArgs& a, int grid, hipStream_t s) {
  const unsigned slices = (unsigned)((a.b + 16 * T - 1) / (16 * T));
  hipLaunchKernelGGL((mfma_kernel<FMT, XT, T, KW>), dim3((unsigned)grid, slices), dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

template <int FMT, int XT, int T>
hipError_t launch_t(const MfmaArgs& a, int kw, int grid, hipStream_t s) {
  if (kw > max_kw(T)) return hipErrorInvalidValue;
  switch (kw) {
    case 1: return launch_kw<FMT, XT, T, 1>(a, grid, s);
    case 2: if constexpr (max_kw(T) >= 2) return launch_kw<FMT, XT, T, 2>(a, grid, s); break;
    case 4: if constexpr (max_kw(T) >= 4) return launch_kw<FMT, XT, T, 4>(a, grid, s); break;
    case 8: if constexpr (max_kw(T) >= 8) return launch_kw<FMT, XT, T, 8>(a, grid, s); break;
  }
  return hipErrorInvalidValue;
}

template <int FMT, int XT>
hipError_t launch_fx(const MfmaArgs& a, int tiles, int kw, int grid, hipStream_t s) {
  switch (tiles) {
    case 1: return launch_t<FMT, XT, 1>(a, kw, grid, s);
    case 2: return launch_t<FMT, XT, 2>(a, kw, grid, s);
    case 4: return launch_t<FMT, XT, 4>(a, kw, grid, s);
    case 8: return launch_t<FMT, XT, 8>(a, kw, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Launch shape of the MFMA kernel for one batch slice of T tiles: K groups, quads per K group and
// per x window, row tiles and workgroups along x.  K groups split K inside a workgroup when N alone
// gives too few workgroups: the smallest KW of 1, 2, 4, 8 that gives at least one workgroup per CU
// (counting the `slices` batch slices), within what the x window holds.
struct MfmaPlan {
  int tiles, kw, qpk, qpp, xrow, ntiles, grid, slices;
};

bool plan_slice(int64_t n, int64_t k, int64_t b, int t, MfmaPlan* p) {
  const int64_t quads = (k + kQuad - 1) / kQuad;
  const int64_t cus = device_cu_count();
  const int slices = (int)((b + 16 * t - 1) / (16 * t));
  const int row_budget = kXBytes / (16 * t);          // window bytes per activation row
  const int max_q = (row_budget - 16) / (kQuad * 2);  // quads per window row, all K groups
  if (max_q < 1) return false;
  int best = 1;
  for (int c = 1; c <= 8; c *= 2) {
    if (c > max_q || c > quads) break;
    best = c;
    const int64_t rows = 16 * (8 / c);
    if ((n + rows - 1) / rows * slices >= cus) break;
  }
  const int64_t per_kg = (quads + best - 1) / best;
  const int per_phase = std::max(1, max_q / best);
  p->tiles = t;
  p->kw = best;
  p->qpk = (int)per_kg;
  p->qpp = (int)std::min<int64_t>(per_kg, per_phase);
  p->xrow = best * p->qpp * kQuad * 2 + 16;
  // Row tiles and workgroups: one workgroup per CU walks several tiles when x fits one window and
  // K is not split (the window and the table are then filled once per workgroup, and each wave's
  // stream of quads runs across its tiles without a pipeline restart); else one per tile.
  const int64_t rows = 16 * (8 / best);
  const int64_t ntile = (n + rows - 1) / rows;
  p->ntiles = (int)ntile;
  p->grid = (best == 1 && p->qpp >= per_kg)
                ? (int)std::min<int64_t>(ntile, std::max<int64_t>(1, cus / slices))
                : (int)ntile;
  p->slices = slices;
  return true;
}

// Batch tiles per slice: the largest T (8, 4, 2, 1; at most what B needs) whose launch has at
// least half a workgroup per CU; slices beyond the first re-read the weights (mostly from L2).
// Byte offsets are 32-bit: a slice's activations (16 T * K * 2 bytes) must stay below 2^31.
bool plan_mfma(int64_t n, int64_t k, int64_t b, MfmaPlan* out) {
  if (b < 1 || b > W4_MAX_BATCH || 16 * kMaxTiles * k * 2 >= ((int64_t)1 << 31)) return false;
  const int64_t cus = device_cu_count();
  const int need = (int)std::min<int64_t>((b + 15) / 16, kMaxTiles);
  const int tmax = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
  bool found = false;
  MfmaPlan best{};
  for (int t = tmax; t >= 1; t /= 2) {
    MfmaPlan p;
    if (!plan_slice(n, k, b, t, &p)) continue;
    if (!found || (int64_t)p.grid * p.slices > (int64_t)best.grid * best.slices) {
      best = p;
      found = true;
    }
    if ((int64_t)p.grid * p.slices * 2 >= cus) {
      best = p;
      break;
    }
  }
  if (found) *out = best;
  return found;
}

// One launch over all B rows of x: grid.y = batch slices of up to 16 T rows.
hipError_t launch_mfma(int fmt, const uint16_t* x, const uint8_t* packed, const void* scales,
                       int64_t n, int64_t k, int64_t b, float* y, hipStream_t s) {
  MfmaPlan p;
  if (!plan_mfma(n, k, b, &p)) return hipErrorNotSupported;
  MfmaArgs a;
  a.x = x;
  a.packed = packed;
  a.scales = scales;
  a.y = y;
  a.n = n;
  a.k = k;
  a.b = (int)b;
  a.qpk = p.qpk;
  a.qpp = p.qpp;
  a.xrow = p.xrow;
  a.tiles = p.ntiles;
  switch (fmt) {
    case W4_NF4_X_F16: return launch_fx<kNF4, kF16>(a, p.tiles, p.kw, p.grid, s);
    case W4_NF4_X_BF16: return launch_fx<kNF4, kBF16>(a, p.tiles, p.kw, p.grid, s);
    case W4_INT4_X_F16: return launch_fx<kINT4, kF16>(a, p.tiles, p.kw, p.grid, s);
    case W4_INT4_X_BF16: return launch_fx<kINT4, kBF16>(a, p.tiles, p.kw, p.grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace w4
