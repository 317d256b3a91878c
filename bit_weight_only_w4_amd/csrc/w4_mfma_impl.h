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
//     are exact in both 16-bit types.  Asymmetric INT4 decodes q - 8 the same way and adds one
//     MFMA per step whose A rows hold -(z - 8), which makes D the block's sum of (q - z) x.
#pragma once
#include <string.h>

#include <algorithm>

#include "w4_mfma_common.h"

namespace w4 {

// One matrix of a launch.  The matrices of a grouped launch share x and K; their row tiles are
// numbered one after another, member g owning tiles [tile0, tile0 + its tiles).
struct MfmaMember {
  const uint8_t* packed;  // [N_g, K/2]
  const void* scales;     // NF4, FP4 float[N_g, K/64] | INT4 uint16 / INT4A uint32 [N_g, K/128]
  float* y;               // [B, N_g]
  uint32_t n;             // N_g
  uint32_t tile0;
};

struct MfmaArgs {
  MfmaMember m[kMaxGroup];
  const uint16_t* x;      // [B, K]
  uint32_t groups;
  uint32_t k;
  uint32_t b;          // activation rows in all; slice blockIdx.y takes rows [16 T y, 16 T (y + 1))
  uint32_t qpk;        // quads per K group
  uint32_t qpp;        // quads per K group in one x window (one phase)
  uint32_t xrow;       // bytes per activation row of the x window: (KW * 32 qpp + 1) * 16
  uint32_t red_bytes;  // LDS bytes of the K-group reduction area (0 when KW == 1)
  uint32_t tiles;      // row tiles (16 RW rows each) in all
  uint32_t tiles_base;  // tiles per workgroup: tiles_base, plus one for blockIdx.x < tiles_rem
  uint32_t tiles_rem;
  uint32_t qps;        // split-K (grid.z > 1): quads per split, KW * qpk; split z owns quads
                       // [z qps, (z + 1) qps) and writes its partial sums to y + z * ysplit
  uint32_t ysplit;     // floats between the partial planes of consecutive splits (B * N)
};

namespace {

constexpr int kThreads = 512;        // 8 waves
constexpr int kLdsBytes = 160 * 1024;  // LDS of a CU: table, reduction area and x window
constexpr int kQuad = 256;          // weights per quad
constexpr int kMaxTiles = 8;        // up to 128 activation rows per launch

// One quad in this lane's registers: 32 packed bytes of the 128-byte quad segments of the tile's
// rows (two 16-byte loads), and the scale of one D row per block: lane (g, m) holds row 4 g + (m & 3),
// and lane (g, n) gets the scales of its rows 4 g + i from lanes (g, i) by a DPP row broadcast.
//   The loads read whole 128-byte lines: load h covers rows 8 h .. 8 h + 7, each row by 8 lanes,
//   its own lanes (g, m) and those of its partner row m ^ 8.  In load h, lane (g, m) takes chunk g
//   of its own row when m >> 3 == h, else chunk g + 4 of the partner row; a DPP rotation by 8
//   lanes swaps the partner chunks when the quad is multiplied, so that lane (g, m) then holds
//   chunks g and g + 4 (bytes [16 g, 16 g + 16) and [64 + 16 g, 80 + 16 g)) of row m.
//   INT4 (2 blocks of 64 bytes): those are bytes [16 g, 16 g + 16) of blocks 0 and 1.
//   NF4 (4 blocks of 32 bytes): bytes [16 g, 16 g + 16) of the 64 bytes of blocks 0, 1 and of
//   blocks 2, 3, so lane groups 0, 1 hold blocks 0 / 2 and groups 2, 3 blocks 1 / 3.  Two
//   v_permlane32_swap give every lane 8 bytes of each block: lane group L then holds the bytes
//   [16 g0, 16 g0 + 8) of both blocks' lane-group-(L & 1) halves, g0 = L & 1, offset by 8 bytes
//   for L >= 2, i.e. the 16 weights from 32 (L & 1) + 16 (L >> 1) of each block.
template <int FMT>
struct Quad {
  static constexpr int QC = is_g128(FMT) ? 2 : 4;  // scale blocks per quad
  uint32_t w[2][4];
  uint32_t s[QC];  // fp32 bits (INT4: bf16 bits in the low half; INT4A: its word)
};

// Waves per SIMD the kernel is compiled for: four (two workgroups per CU, <= 128 VGPRs) for one
// batch tile, two above.
constexpr int min_waves(int t) { return t == 1 ? 4 : 2; }

template <int FMT, int XT, int T, int KW, bool GROUPED>
__global__ void __launch_bounds__(kThreads, min_waves(T)) mfma_kernel(MfmaArgs a) {
  constexpr int RW = 8 / KW;
  constexpr int KC = is_g128(FMT) ? 128 : 64;  // weights per scale block
  constexpr int QC = kQuad / KC;              // blocks per quad
  constexpr int STEPS = KC / 32;              // MFMA steps per block
  constexpr int SB = FMT == kINT4 ? 2 : 4;     // bytes per scale
  constexpr bool kSplit = (FMT == kNF4 && XT == kBF16);
  // LDS: the decode table (static, at address 0, so a lookup address needs no base), then the
  // dynamic part: the K-group reduction area and the x window.
  __shared__ __align__(16) uint32_t tab[kTableBytes / 4];
  extern __shared__ __align__(16) uint8_t smem[];
  float4_t* red = reinterpret_cast<float4_t*>(smem);  // [KW - 1][RW][T][64 lanes]
  uint8_t* xs = smem + a.red_bytes;

  // The wave index through readfirstlane: everything derived from it stays in scalar registers.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % RW, kg = wave / RW;
  const int g = lane >> 4, m = lane & 15;
  const uint32_t k = a.k;
  const uint32_t nblocks = k / KC;
  const uint32_t pitch = k >> 1;
  const uint32_t spitch = nblocks * SB;
  // This workgroup's batch slice: activation rows [16 T y, 16 T y + bsl); the window holds them.
  const uint32_t b0 = blockIdx.y * 16u * T;
  const uint32_t bsl = min(16u * T, a.b - b0);
  const uint16_t* xsl = a.x + (size_t)b0 * k;
  // Split-K: this workgroup's first quad of K (0 without a split).
  const uint32_t zq = blockIdx.z * a.qps;
  const __amdgpu_buffer_rsrc_t rx_ = make_rsrc(xsl, bsl * k * 2u);

  // The workgroup's row tiles: blockIdx.x, blockIdx.x + gridDim.x, ... (ntiles of them).
  const int ntiles = (int)(a.tiles_base + (blockIdx.x < a.tiles_rem ? 1u : 0u));
  const int nq = (int)a.qpk;         // quads per tile and wave
  const int len = ntiles * nq;       // this wave's stream of (tile, quad) positions

  // Per-lane byte offsets inside a row tile: the A bytes of row m / lane group g, and the scale
  // row 4 g + (m & 3) (see Quad).
  // This lane's two weight loads (see Quad): row and 16-byte chunk inside the quad segment.
  const int chunk0 = m < 8 ? g : g + 4, chunk1 = m < 8 ? g + 4 : g;
  const uint32_t wl0 = (uint32_t)(m & 7) * pitch + (uint32_t)(chunk0 * 16);
  const uint32_t wl1 = (uint32_t)(8 + (m & 7)) * pitch + (uint32_t)(chunk1 * 16);
  const uint32_t wblk0 = (uint32_t)(chunk0 / (KC / 32)), wblk1 = (uint32_t)(chunk1 / (KC / 32));
  const uint32_t slane = (uint32_t)(4 * g + (m & 3)) * spitch;

  // A cursor over this wave's stream of (tile ti, quad q) positions, with the buffer resources of
  // tile ti's 16 rows (rows past N, and tiles past the stream, read as zero).
  struct Cursor {
    int ti, q;
    __amdgpu_buffer_rsrc_t rw, rs;
  };
  // The member that owns global tile t (uniform), by selects over the fixed member slots so that
  // the argument block is never indexed dynamically.
  auto member = [&](uint32_t t) __attribute__((always_inline)) {
    MfmaMember r = a.m[0];
    if constexpr (GROUPED) {
#pragma unroll
      for (int i = 1; i < kMaxGroup; ++i) {
        if ((uint32_t)i < a.groups && t >= a.m[i].tile0) r = a.m[i];
      }
    }
    return r;
  };
  auto set_tile = [&](Cursor& c) __attribute__((always_inline)) {
    const uint32_t tg = blockIdx.x + (uint32_t)c.ti * gridDim.x;
    const MfmaMember mm = member(tg);
    const uint32_t row_base = ((tg - mm.tile0) * RW + rg) * 16u;
    const uint32_t rows_left = c.ti < ntiles && row_base < mm.n ? mm.n - row_base : 0u;
    const uint32_t rows = rows_left >= 16u ? 16u : rows_left;
    c.rw = make_rsrc(mm.packed + (size_t)row_base * pitch, rows * pitch);
    c.rs = make_rsrc(reinterpret_cast<const char*>(mm.scales) + (size_t)row_base * spitch, rows * spitch);
  };
  // The resources change only at a new tile (a uniform branch).
  auto advance = [&](Cursor& c) __attribute__((always_inline)) {
    const bool wrap = c.q + 1 == nq;
    c.q = wrap ? 0 : c.q + 1;
    if (wrap) {
      c.ti += 1;
      set_tile(c);
    }
  };
  // The quad at the cursor: blocks qb .. qb + QC - 1 of the K group,
// qb = (z qps + kg * qpk + q) * QC.
  // Blocks past K read as zero (their weights and scales), which adds nothing.  Each lane's 16
  // bytes lie inside one block.
  auto load_quad = [&](const Cursor& cur, Quad<FMT>& d) __attribute__((always_inline)) {
    const uint32_t qb = (zq + (uint32_t)kg * a.qpk + (uint32_t)cur.q) * QC;
    const uint32_t wq = qb * (KC / 2);  // byte offset of the quad segment in a row
    const uint32_t sbase = slane + qb * SB;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bool have = qb + (h ? wblk1 : wblk0) < nblocks;
      const uint4 v = buffer_load16_stream(cur.rw, offset_or_oob(have, (h ? wl1 : wl0) + wq));
      d.w[h][0] = v.x;
      d.w[h][1] = v.y;
      d.w[h][2] = v.z;
      d.w[h][3] = v.w;
    }
    // NF4: the quad's four fp32 scales of this lane's row are contiguous (dword aligned), one
    // 16-byte load; of a quad that ends past K, the blocks past K are zeroed when the quad is
    // multiplied (inside the matrix their bytes are the next row's; zeroing them here would make
    // the loop wait for the load).  INT4: two bf16 scales, 2-byte aligned, two loads, moved to the
    // high half when multiplied (for the same reason).
    if constexpr (!is_g128(FMT)) {
      const uint4 sv = buffer_load16(cur.rs, offset_or_oob(qb < nblocks, sbase));
      d.s[0] = sv.x;
      d.s[1] = sv.y;
      d.s[2] = sv.z;
      d.s[3] = sv.w;
    } else {
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const bool have = qb + c < nblocks;
        const uint32_t off = offset_or_oob(have, sbase) + (uint32_t)(c * SB);
        d.s[c] = FMT == kINT4A ? buffer_load32(cur.rs, off) : buffer_load16bit(cur.rs, off);
      }
    }
  };

  // x window of phase p: for every batch row r < bsl and K group kk, the quads
  // z qps + kk * qpk + p * qpp .. + qpp - 1 that the K group has (other pieces read as zero).  The window
  // is copied straight from global memory into LDS (buffer loads with the LDS destination): the
  // 16-byte slot s = base + tid receives thread tid's load, so slot s holds piece
  // col = s % P of row r = s / P, P = KW * seg + 1 pieces per row, the last one padding (it puts
  // consecutive rows four banks apart).  Only the slots of the bsl rows are loaded.
  const uint32_t seg = a.qpp * 32u;  // 16-byte pieces of one K group's segment of a row
  const uint32_t P = (uint32_t)KW * seg + 1u;
  const uint32_t slots = bsl * P;
  const uint32_t nphase = (a.qpk + a.qpp - 1) / a.qpp;
  // Row of slot s and K group of piece col through float reciprocals: with the + 0.5 offset,
  // (s + 0.5) / P is at least 1 / (2 P) away from an integer, and bsl * P <= 8192 (the window fits
  // 128 KiB) keeps the fp32 error, at most bsl * 2^-23, far below that; likewise (col + 0.5) / seg
  // (error at most KW * 2^-23, margin 1 / (2 seg) >= 2^-14).
  const float inv_p = 1.0f / (float)P;
  const float inv_seg = 1.0f / (float)seg;
  auto load_x = [&](uint32_t p) __attribute__((always_inline)) {
    const uint32_t q0 = p * a.qpp;  // first quad of the phase inside each K group
    for (uint32_t base = 0; base < slots; base += kThreads) {
      uint32_t sl = base + (uint32_t)tid;
      asm volatile("" : "+v"(sl));
      const uint32_t r = (uint32_t)(((float)sl + 0.5f) * inv_p);
      const uint32_t col = sl - r * P;
      const uint32_t kk = (uint32_t)(((float)col + 0.5f) * inv_seg);
      const uint32_t pc = col - kk * seg;
      const uint32_t ql = q0 + (pc >> 5);  // quad inside the K group
      const uint32_t kpos = (zq + kk * a.qpk + ql) * kQuad + (pc & 31u) * 8u;
      const bool have = sl < slots && kk < (uint32_t)KW && ql < a.qpk && kpos < k;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx_, (__attribute__((address_space(3))) void*)(xs + (base + (uint32_t)wave * 64u) * 16u), 16,
          (int)offset_or_oob(have, (r * k + kpos) * 2u), 0, 0, 0);
    }
  };

  // The load cursor runs R positions ahead of the compute cursor (R register sets; two for 8
  // batch tiles, whose accumulators leave no room for four).
  constexpr int R = T == 8 ? 2 : 4;
  Cursor ld;
  ld.ti = 0;
  ld.q = 0;
  set_tile(ld);
  // Prologue order: the window's buffer-to-LDS loads first, then the weight quads, then the
  // table, then the barrier.  Memory operations complete in issue order, so what waits for the
  // window (the table's LDS stores, which the compiler cannot tell apart from the window's, and
  // the barrier) waits for it alone, not for the weights behind it: no wave holds the barrier for
  // its own HBM loads, and all four quads are in flight across it.  (Weights first and the window
  // last made the barrier wait for every load in flight; the table first delayed the weights.)
  Quad<FMT> P0, P1, P2, P3;
  load_x(0);
  load_quad(ld, P0);
  advance(ld);
  load_quad(ld, P1);
  advance(ld);
  fill_table<FMT, XT, kThreads>(tab);
  if constexpr (R == 4) {
    load_quad(ld, P2);
    advance(ld);
    load_quad(ld, P3);
    advance(ld);
  }
  __syncthreads();

  float4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Twice this lane's byte offset in a table entry (see the lookup below).
  const uint32_t laneoff = kSplit ? (uint32_t)(lane & 15) * 16u : (uint32_t)(lane & 31) * 8u;
  const char* tabc = reinterpret_cast<const char*>(tab);
  const uint8_t* xw = xs + (uint32_t)kg * (seg * 16u);  // this K group's part of the window

  // k offset (in the block) of the first of this lane's weights for MFMA step 0 (see Quad).
  const int klane = !is_g128(FMT) ? 32 * (g & 1) + 16 * (g >> 1) : 32 * g;
  // INT4A: the lane holding the scale word of A row m (scale words sit with D rows 4 g + (m & 3)).
  const int zsrc = 16 * (m >> 2) + (m & 3);

  // Multiply the quad held in d: quad q of the K group, wq = its index inside the current window.
  auto compute = [&](int q, int wq, const Quad<FMT>& d) __attribute__((always_inline)) {
    const uint32_t qb = (zq + (uint32_t)kg * a.qpk + (uint32_t)q) * QC;  // its first scale block
    // this lane's 2 (NF4) or 4 (INT4) dwords of packed bytes per block
    // Chunks g and g + 4 of row m: keep the own one, take the partner's by a rotation of 8 lanes.
    uint32_t wh[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t send = m < 8 ? d.w[1][i] : d.w[0][i];
      wh[0][i] = m < 8 ? d.w[0][i] : d.w[1][i];
      wh[1][i] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0x128, 0xF, 0xF, false);  // row_ror:8
    }
    uint32_t wb[QC][STEPS];
    if constexpr (!is_g128(FMT)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const auto s0 = __builtin_amdgcn_permlane32_swap(wh[h][0], wh[h][2], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(wh[h][1], wh[h][3], false, false);
        wb[2 * h][0] = s0[0];
        wb[2 * h][1] = s1[0];
        wb[2 * h + 1][0] = s0[1];
        wb[2 * h + 1][1] = s1[1];
      }
    } else {
#pragma unroll
      for (int c = 0; c < QC; ++c) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s) wb[c][s] = wh[c][s];
      }
    }
    const uint8_t* xq = xw + (wq * kQuad + klane) * 2;
    // This lane's B rows: activation row 16 t + m of the slice, or the last one held when the
    // slice is shorter (those columns of D are never stored).  Recomputed per quad (the opaque
    // copy of the limit keeps the compiler from holding T offsets across the main loop).
    uint32_t blim = bsl - 1u;
    asm volatile("" : "+s"(blim));
    uint32_t xrowoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t) xrowoff[t] = min((uint32_t)(16 * t + m), blim) * a.xrow;
#pragma unroll
    for (int c = 0; c < QC; ++c) {
      float4_t dd[T];
#pragma unroll
      for (int t = 0; t < T; ++t) dd[t] = float4_t{0.f, 0.f, 0.f, 0.f};
      // INT4A: A operand whose row m is -(z_m - 8) everywhere; its product with the block's x adds
      // -(z - 8) * sum(x) to D, turning the decoded codes q - 8 into q - z.
      uint4 zrow = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (FMT == kINT4A) {
        const uint32_t word = (uint32_t)__shfl((int)d.s[c], zsrc);
        const float zn = (float)(8 - (int)((word >> 16) & 15u));
        const uint32_t h = XT == kF16 ? f16_bits(zn) : (__float_as_uint(zn) >> 16);
        const uint32_t hh = h | (h << 16);
        zrow = make_uint4(hh, hh, hh, hh);
      }
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
          const uint4 bv = *reinterpret_cast<const uint4*>(xq + xrowoff[t] + (c * KC + s * 8) * 2);
          dd[t] = mfma<XT>(a1, bv, dd[t]);
          if (kSplit) dd[t] = mfma<XT>(make_uint4(p2[0], p2[1], p2[2], p2[3]), bv, dd[t]);
          if (FMT == kINT4A) dd[t] = mfma<XT>(zrow, bv, dd[t]);
        }
        // With 8 tiles, keep each step's B fragments from being fetched ahead of the previous
        // step (they would not fit the registers left by the accumulators).
        if constexpr (T == 8) __builtin_amdgcn_sched_barrier(0);
      }
      const uint32_t sraw = !is_g128(FMT) ? ((c > 0 && qb + c >= nblocks) ? 0u : d.s[c]) : d.s[c] << 16;
      const float sc[4] = {row_bcast<0>(sraw), row_bcast<1>(sraw), row_bcast<2>(sraw),
                           row_bcast<3>(sraw)};
#pragma unroll
      for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = __builtin_fmaf(dd[t][i], sc[i], acc[t][i]);
      }
    }
  };

  // y rows of tile ti: after its last quad, K groups add up in the reduction area (KW > 1) and
  // kg == 0 stores; lane (g, m) holds y[16 t + m][row_d + i], i = 0..3.
  auto finish_tile = [&](int ti) __attribute__((always_inline)) {
    const uint32_t tg = blockIdx.x + (uint32_t)ti * gridDim.x;
    const MfmaMember mm = member(tg);
    const uint32_t n = mm.n;
    const uint32_t row_d = ((tg - mm.tile0) * RW + rg) * 16u + 4u * g;
    float* ysl = mm.y + (size_t)blockIdx.z * a.ysplit + (size_t)b0 * n;
    if constexpr (KW > 1) {
      __syncthreads();  // the previous tile's sums have been read
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
        const uint32_t b = 16u * t + m;
        if (b < bsl) {
          float* yr = ysl + (size_t)b * n;
          if ((n & 3u) == 0 && row_d + 3 < n) {
            // the lane's four rows are consecutive in y: one 16-byte store
            *reinterpret_cast<float4_t*>(yr + row_d) = acc[t];
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (row_d + i < n) yr[row_d + i] = acc[t][i];
            }
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  };

  // One stream position with the quad in d: a new x window at every multiple of qpp quads when a
  // K group needs several windows (also back to phase 0 at each new tile), the multiply, the
  // refill of d R positions ahead, and the end of the tile after its last quad.
  int ct = 0, cq = 0;
  auto step = [&](Quad<FMT>& d) __attribute__((always_inline)) {
    if (nphase > 1 && (cq > 0 || ct > 0) && cq % a.qpp == 0) {
      __syncthreads();  // every wave is done with the old window
      load_x((uint32_t)cq / a.qpp);
      // The window's copies are this wave's last loads: wait for all of them, since the barrier
      // does not wait for the copies of other waves.
      wait_all_vector_loads();
      __syncthreads();
    }
    compute(cq, nphase > 1 ? cq % (int)a.qpp : cq, d);
    load_quad(ld, d);
    advance(ld);
    const bool last = cq == nq - 1;
    if (last) finish_tile(ct);
    ct += last ? 1 : 0;
    cq = last ? 0 : cq + 1;
  };

  // Main loop: R positions per trip, the register sets rotating without copies; the last
  // positions are already loaded when it ends.
  int j = 0;
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

// K groups instantiated for T batch tiles: 8 / 4 / 2 / 1.
constexpr int max_kw(int t) { return t == 1 ? 8 : t == 2 ? 4 : t == 4 ? 2 : 1; }

// Workgroups of one instantiation that fit a CU with `lds` bytes of dynamic LDS (registers and
// LDS), from the runtime; the dynamic LDS limit is raised once per instantiation.
template <int FMT, int XT, int T, int KW, bool GROUPED>
int resident_kw(int lds) {
  static bool raised = false;
  if (!raised) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&mfma_kernel<FMT, XT, T, KW, GROUPED>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes - kTableBytes);
    raised = true;
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &nb, reinterpret_cast<const void*>(&mfma_kernel<FMT, XT, T, KW, GROUPED>), kThreads, lds) !=
      hipSuccess)
    return 0;
  return nb;
}

template <int FMT, int XT, int T, int KW, bool GROUPED>
hipError_t launch_kw(const MfmaArgs& a, int lds, int grid, int slices, hipStream_t s) {
  const uint32_t quads = (a.k + kQuad - 1) / kQuad;
  const uint32_t splits = a.qps ? (quads + a.qps - 1) / a.qps : 1u;
  hipLaunchKernelGGL((mfma_kernel<FMT, XT, T, KW, GROUPED>),
                     dim3((unsigned)grid, (unsigned)slices, (unsigned)splits), dim3(kThreads),
                     (unsigned)lds, s, a);
  return hipGetLastError();
}

// Instantiation dispatch: op 0 = resident workgroups per CU (returned in *out), op 1 = launch.
template <int FMT, int XT, int T, bool GROUPED>
hipError_t dispatch_t(int op, const MfmaArgs& a, int kw, int lds, int grid, int slices, int* out,
                      hipStream_t s) {
  if (kw > max_kw(T)) return hipErrorInvalidValue;
#define W4_MFMA_KW(KWV)                                                    \
  if (kw == KWV) {                                                         \
    if constexpr (max_kw(T) >= KWV) {                                      \
      if (op == 0) {                                                       \
        *out = resident_kw<FMT, XT, T, KWV, GROUPED>(lds);                          \
        return hipSuccess;                                                 \
      }                                                                    \
      return launch_kw<FMT, XT, T, KWV, GROUPED>(a, lds, grid, slices, s);          \
    }                                                                      \
  }
  W4_MFMA_KW(1)
  W4_MFMA_KW(2)
  W4_MFMA_KW(4)
  W4_MFMA_KW(8)
#undef W4_MFMA_KW
  return hipErrorInvalidValue;
}

template <int FMT, int XT, bool GROUPED>
hipError_t dispatch_fx(int op, const MfmaArgs& a, int tiles, int kw, int lds, int grid, int slices,
                       int* out, hipStream_t s) {
  switch (tiles) {
    case 1: return dispatch_t<FMT, XT, 1, GROUPED>(op, a, kw, lds, grid, slices, out, s);
    case 2: return dispatch_t<FMT, XT, 2, GROUPED>(op, a, kw, lds, grid, slices, out, s);
    case 4: return dispatch_t<FMT, XT, 4, GROUPED>(op, a, kw, lds, grid, slices, out, s);
    case 8: return dispatch_t<FMT, XT, 8, GROUPED>(op, a, kw, lds, grid, slices, out, s);
  }
  return hipErrorInvalidValue;
}

template <bool GROUPED>
hipError_t dispatch(int op, int fmt, const MfmaArgs& a, int tiles, int kw, int lds, int grid,
                    int slices, int* out, hipStream_t s) {
  switch (fmt) {
    case W4_NF4_X_F16: return dispatch_fx<kNF4, kF16, GROUPED>(op, a, tiles, kw, lds, grid, slices, out, s);
    case W4_NF4_X_BF16: return dispatch_fx<kNF4, kBF16, GROUPED>(op, a, tiles, kw, lds, grid, slices, out, s);
    case W4_INT4_X_F16: return dispatch_fx<kINT4, kF16, GROUPED>(op, a, tiles, kw, lds, grid, slices, out, s);
    case W4_INT4_X_BF16: return dispatch_fx<kINT4, kBF16, GROUPED>(op, a, tiles, kw, lds, grid, slices, out, s);
    case W4_FP4_X_F16: return dispatch_fx<kFP4, kF16, GROUPED>(op, a, tiles, kw, lds, grid, slices, out, s);
    case W4_FP4_X_BF16: return dispatch_fx<kFP4, kBF16, GROUPED>(op, a, tiles, kw, lds, grid, slices, out, s);
    case W4_INT4A_X_F16: return dispatch_fx<kINT4A, kF16, GROUPED>(op, a, tiles, kw, lds, grid, slices, out, s);
    case W4_INT4A_X_BF16: return dispatch_fx<kINT4A, kBF16, GROUPED>(op, a, tiles, kw, lds, grid, slices, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Op 0 (resident workgroups per CU) or op 1 (launch) of the grouped instantiations, which live in
// their own translation unit.
hipError_t mfma_dispatch_grouped(int op, int fmt, const MfmaArgs& a, int tiles, int kw, int lds,
                                 int grid, int slices, int* out, hipStream_t s);

}  // namespace w4
