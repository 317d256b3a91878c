// Prefill-size GEMM for fp16 activations with the block scale folded into the decoded weights:
// y[m, n] = sum_k x[m, k] * W_hat[n, k], W_hat[n, k] = code(q[n, k]) * s[n, block(k)].
//
// Prefill needs a GEMM, not a GEMV per token (LLM Quantization on RTX 4060, "Why Only 16%", item
// 3).  The block-scale kernel (w4_gemm.hip) multiplies the raw codes on the matrix cores and
// rescales every block's fresh fp32 partial sums by the block scale: one FMA per output per 64
// weights, about as many vector instructions as the matrix cores spend cycles.  With fp16
// activations the decoded weight itself can be formed in fp16 instead: the table gives the code in
// fp16, one packed multiply per pair applies the fp16-rounded scale, and the matrix cores then
// accumulate x * W_hat across all blocks directly.  The rounding stays inside the accuracy bound
// (|y - y_exact| <= 2e-3 sum_k |x w_hat| + 1e-5): code, scale and product each round to fp16
// (at most 2^-11 relative each), so a folded NF4 weight is within 3 * 2^-11 = 1.5e-3 of W_hat,
// an FP4 weight (exact code) within 2 * 2^-11, an INT4 weight, (q - 8) s with a bf16 scale
// (at most 3 + 8 significant bits), is exact, and an asymmetric INT4 weight, (q - z) s formed as
// ((q - 8) + (8 - z)) s (the sum an exact small integer, at most 4 + 8 significant bits in the
// product), is within 2^-11.  The products with fp16 x are exact in fp32.
//
// A folded weight must stay a normal, finite fp16 number: a block whose scale s satisfies
// lo <= |s| <= hi (or s == 0) is folded, with [lo, hi] = [2^-10, 2^15] for NF4 (smallest nonzero
// |code| 0.0796), [2^-13, 2^13] for FP4 (codes 0.5 .. 6), [2^-14, 2^12] for INT4 (|q - 8| <= 8)
// and asymmetric INT4 (|q - z| <= 15: at most 61440).
// Every wave checks all block scales of its rows once, in its prologue; a wave that meets one
// outside that range (tiny, huge, infinite or NaN scales) runs all of K through the block-scale
// route instead: raw codes on the matrix cores, fp32 rescaling of each block's partial sums.
//
// Work layout.  A workgroup has 4 waves and an output tile of TN = 128 NT weight rows x TM = 128
// activation rows (32 for the slices below); wave w owns weight rows [32 NT w, 32 NT (w + 1)) of
// the tile and all TM activation rows, so every weight is decoded once per tile.  Matrix step:
// v_mfma_f32_32x32x16_f16
// with the activations as the A operand and the weights as the B operand:
//   * A (32 activation rows x 16 k): lane l = 32 h + c takes row c and 8 consecutive k.
//   * B (16 k x 32 weight rows): lane l = 32 h + c takes weight row c and the same 8 k.
//   * D (32 x 32 fp32, 16 registers): lane l = 32 h + c holds weight row c, activation rows
//     8 (e / 4) + 4 h + e % 4 (register e).  Each lane's outputs share one weight row, so a block
//     scale reaches them without any cross-lane broadcast.
// K runs one 64-weight block per step (an NF4/FP4 block, half an INT4 group).  Asymmetric INT4
// decodes q - 8 through INT4's table and adds 8 - z (one packed add per pair) before the scale.  Lane (h, c) loads
// bytes [16 h, 16 h + 16) of its row's 32-byte block: weights 32 h .. 32 h + 31, of which matrix
// step q (0 .. 3) takes 32 h + 8 q .. + 7; the A lanes read the same k positions of x.
//   * Activations: ST stages of TM rows x 64 k in LDS (16 KiB each), copied straight from global
//     memory by buffer loads with the LDS destination (no register round trip), ST - 1 blocks
//     ahead; 16-byte slot S of a stage holds row S / 8 and chunk (S % 8) XOR ((row / 2) % 8), which
//     puts the sixteen rows a 16-lane group reads into distinct banks (see xkey).
//   * Weights and scales: DP blocks ahead in rotating register sets.
//   * Decode: the byte -> pair table of w4_mfma_common.h (32 copies, one LDS read per two weights);
//     FP4 converts in registers instead (gfx950 E2M1 conversion, no table).
//   * Tiles are numbered so that the workgroups one XCD receives (every eighth) take consecutive
//     tiles, the activation-row tiles of a weight tile first: the weight tile then comes from that
//     XCD's L2 after its first read.
//   * K may be split into ranges of whole blocks (grid.y; an even number of blocks for INT4, so a
//     range starts on a group): a workgroup addresses the weights, scales and activations from its
//     range's first block on, with the matrix's row pitches, and writes fp32 partial sums to its
//     range's plane; a second kernel adds the planes in range order (fixed-order, reproducible).
//   * A one-pass launch whose tiles leave a sparse last round (see launch_gemm_fold) runs that
//     round as a second launch of 32-row slices (TM = 32, four workgroups per tile): each weight
//     of such a tile is decoded four times, but the round spreads over the whole chip, and every
//     output's sum over K runs in the same order as in a full tile.
#include <algorithm>

#include "w4_mfma_common.h"

namespace w4 {

struct FoldMember {
  const uint8_t* packed;  // [N_g, K/2]
  const void* scales;     // NF4, FP4 float[N_g, K/64] | INT4 uint16 (bf16) [N_g, K/128]
  float* y;               // [M, N_g]
  uint32_t n;             // N_g
  uint32_t tile0;         // first tile of this member
};

struct FoldArgs {
  FoldMember mb[kMaxGroup];
  const uint16_t* x;  // [M, K] fp16 bits
  uint32_t groups;
  uint32_t m, k;
  uint32_t mt;     // activation-row tiles (128 rows each)
  uint32_t tiles;  // workgroups along x: tiles of this launch times the slices of each
  uint32_t tile_base;  // first tile of this launch (tiles counted over all members)
  uint32_t bps;    // 64-weight blocks per K range: range z = blockIdx.y owns blocks
                   // [z bps, min((z + 1) bps, K / 64)) and writes y + z * ysplit
  uint32_t ysplit; // floats between the partial planes of consecutive ranges (M * N; one member)
};

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kFoldThreads = 256;
constexpr int kFoldMT = 4;  // 32-row activation tiles per wave in a full tile: TM = 128
constexpr int kWideMT = 6;  // the 192-row tile, for 129 to 192 activation rows

__device__ inline f32x16 mfma32(const uint4& a, const uint4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                 __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// XOR key of the 16-byte chunks of activation row mr in a stage: (mr / 2) mod 8.  A 128-bit LDS
// read serves 16 lanes per cycle across 64 banks (16 slots); the 16 lanes of a fragment read take
// rows r .. r + 15 at one chunk, whose slots must then differ mod 16: row parity gives slot bit 3,
// the key bits 0-2 (a key of mr mod 8 repeats for rows r and r + 8: two-way conflicts).
__device__ inline uint32_t xkey(uint32_t mr) { return (mr >> 1) & 7u; }

// The fold range of a block scale (see the top of this file), and the scale as fp32.
template <int FMT>
__device__ inline bool foldable(float s) {
  const float a = __builtin_fabsf(s);
  constexpr float lo = FMT == kNF4 ? 0x1p-10f : FMT == kFP4 ? 0x1p-13f : 0x1p-14f;
  constexpr float hi = FMT == kNF4 ? 0x1p15f : FMT == kFP4 ? 0x1p13f : 0x1p12f;
  return s == 0.0f || (a >= lo && a <= hi);
}
// raw: the scale as stored (NF4, FP4: fp32; INT4: bf16 in the low half; asymmetric INT4: the
// group's 32-bit word, bf16 scale low, zero point in bits 16-19).
template <int FMT>
__device__ inline float scale_f32(uint32_t raw) {
  return is_g128(FMT) ? __uint_as_float(raw << 16) : __uint_as_float(raw);
}
// Asymmetric INT4: 8 - z as an fp16 pair, which turns the table's q - 8 into q - z (small
// integers: exact).
__device__ inline uint32_t zero_shift_pair(uint32_t word) {
  const _Float16 d = (_Float16)(8.0f - (float)((word >> 16) & 15u));
  return __builtin_bit_cast(uint32_t, half2_t{d, d});
}

// The four weight pairs of packed dword wd (byte j: weight 2j in the high nibble, 2j + 1 in the
// low one) as unscaled fp16 codes, weight 2j in the low half.  NF4 and INT4 through the LDS table:
// one read per byte at byte * 128 + the lane's copy offset (the perm builds byte * 256 + 2 * copy
// offset, the packed byte into byte 1, halved by the shift).  FP4 through gfx950's E2M1
// conversion instead (one instruction per byte, exact, no table): it puts the low nibble in the
// low half, so the nibbles of every byte are swapped first.
template <int FMT>
__device__ inline void decode4(uint32_t wd, const char* tabc, uint32_t laneoff, uint32_t (&p)[4]) {
  if constexpr (FMT == kFP4) {
    const uint32_t sw = ((wd >> 4) & 0x0F0F0F0Fu) | ((wd & 0x0F0F0F0Fu) << 4);
    p[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(sw, 1.0f, 0));
    p[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(sw, 1.0f, 1));
    p[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(sw, 1.0f, 2));
    p[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(sw, 1.0f, 3));
  } else {
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
      const uint32_t addr =
          __builtin_amdgcn_perm(wd, laneoff, 0x0C0C0000u | ((4u + (uint32_t)kb4) << 8)) >> 1;
      p[kb4] = *reinterpret_cast<const uint32_t*>(tabc + addr);
    }
  }
}

// The block-scale route of one wave, for rows that hold a scale outside the fold range: raw codes
// on the matrix cores, each block's partial sums rescaled in fp32 (exact scale, any range), then
// the wave's stores.  It walks the same stages with the same barriers as the folded loop (the
// stages are filled by every wave of the workgroup) but loads each block's weights when it needs
// them.  Kept out of line, with accumulators of its own: the folded loop's registers are then
// allocated as if this route did not exist (inlined, it cost the folded route 8-30%).
template <int FMT, int NT, int MT>
__device__ __attribute__((noinline)) void fold_block_scale_wave(
    __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rx,
    const char* tabc, uint4* xs0, uint4* xs1, float* y, uint32_t n, uint32_t m, uint32_t m0,
    uint32_t wrow0, uint32_t k, uint32_t nkb) {
  constexpr int ST = 2;
  constexpr int SLOTS = 32 * MT * 8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c = lane & 31;
  const uint32_t pitch = k >> 1;  // k: the row pitch; nkb: the blocks of this K range
  constexpr uint32_t kSB = FMT == kINT4 ? 2u : 4u;
  const uint32_t spitch = (k / (is_g128(FMT) ? 128u : 64u)) * kSB;
  const uint32_t laneoff = (uint32_t)c * 8u;
  f32x16 acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][j][e] = 0.f;
  for (uint32_t kb = 0; kb < nkb; ++kb) {
    const uint32_t b = kb % (uint32_t)ST;
    uint4* const xst = b ? xs1 : xs0;
    wait_own_stage_copies(xst + tid);
    __syncthreads();
    {
      const uint32_t kn = kb + ST - 1, bn = (b + ST - 1) % ST;
      const bool have = kn < nkb;
#pragma unroll
      for (int j = 0; j < SLOTS / kFoldThreads; ++j) {
        const uint32_t sl = (uint32_t)(j * kFoldThreads + tid);
        const uint32_t mr = sl >> 3, cc = (sl & 7u) ^ xkey(mr);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (__attribute__((address_space(3))) void*)((bn ? xs1 : xs0) + j * kFoldThreads + wave * 64),
            16, (int)offset_or_oob(have, (mr * k + kn * 64u + cc * 8u) * 2u), 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t row = (uint32_t)(32 * t + c);
      const uint4 w = buffer_load16_stream(rw, row * pitch + kb * 32u + 16u * (uint32_t)h);
      const uint32_t raw = FMT == kINT4    ? buffer_load16bit(rs, row * spitch + (kb >> 1) * 2u)
                           : FMT == kINT4A ? buffer_load32(rs, row * spitch + (kb >> 1) * 4u)
                                           : buffer_load32(rs, row * spitch + kb * 4u);
      const float sf = scale_f32<FMT>(raw);
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
      uint4 bu[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t pr[4];
        decode4<FMT>(wd[q], tabc, laneoff, pr);
        if constexpr (FMT == kINT4A) {
          const half2_t zz = __builtin_bit_cast(half2_t, zero_shift_pair(raw));
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pr[e] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pr[e]) + zz);
        }
        bu[q] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
      }
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        f32x16 dd;
#pragma unroll
        for (int e = 0; e < 16; ++e) dd[e] = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t mr = (uint32_t)(32 * j + c), cc = (uint32_t)(4 * h + q);
          dd = mfma32(xst[mr * 8u + (cc ^ xkey(mr))], bu[q], dd);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][j][e] = __builtin_fmaf(dd[e], sf, acc[t][j][e]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t col = wrow0 + 32u * t + (uint32_t)c;
    if (col >= n) continue;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t mr = m0 + 32u * j + 8u * (uint32_t)(e >> 2) + 4u * (uint32_t)h + (uint32_t)(e & 3);
        if (mr < m) y[(size_t)mr * n + col] = acc[t][j][e];
      }
    }
  }
}

template <int FMT, int NT, int MT, int ST, int DP, bool GROUPED>
__global__ void __launch_bounds__(kFoldThreads, 2) fold_kernel(FoldArgs a) {
  constexpr int TN = 4 * 32 * NT, TM = 32 * MT;
  // activation rows of the tile grid: 128 (whole tiles or slices of them), or 192 in one tile
  constexpr int FULL = MT > kFoldMT ? MT : kFoldMT;
  constexpr uint32_t SUBS = FULL / MT;  // slices of TM activation rows per tile of the grid
  constexpr int SLOTS = TM * 8;  // 16-byte slots of one stage (64 k per row)
  // the byte -> pair table (not used by FP4, which converts in registers)
  __shared__ __align__(16) uint32_t tab[FMT == kFP4 ? 4 : kTableBytes / 4];
  // The two stages are separate LDS objects and every access names one of them statically: the
  // compiler then tells a stage's reads from the copies into the other stage (and from the table)
  // and waits only for the copies a read depends on.  As one array indexed by stage, every LDS read
  // (table lookups included) waited for all copies in flight, the next stage's too: one round trip
  // per block.
  static_assert(ST == 2, "two stages, each its own LDS object");
  __shared__ __align__(16) uint4 xs0[SLOTS];
  __shared__ __align__(16) uint4 xs1[SLOTS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, c = lane & 31;

  const uint32_t id = blockIdx.x, units = a.tiles;
  const uint32_t xcd = id % 8u, per = units / 8u, extra = units % 8u;
  const uint32_t unit = xcd * per + min(xcd, extra) + id / 8u;
  const uint32_t tile = a.tile_base + unit / SUBS, sub = unit % SUBS;
  FoldMember mm = a.mb[0];
  if constexpr (GROUPED) {
#pragma unroll
    for (int i = 1; i < kMaxGroup; ++i) {
      if ((uint32_t)i < a.groups && tile >= a.mb[i].tile0) mm = a.mb[i];
    }
  }
  const uint32_t lt = tile - mm.tile0;
  const uint32_t tn = lt / a.mt, tm = lt - tn * a.mt;
  const uint32_t m0 = tm * (32u * FULL) + sub * TM;
  if (m0 >= a.m) return;  // a slice past the last activation row: the whole workgroup, no barrier
  // This workgroup's K range, blocks [kb_lo, kb_lo + nkb): weights, scales and activations are
  // addressed from block kb_lo on (block kb below is block kb_lo + kb of the row); k stays the
  // row pitch.  Each resource ends where the matrix does.
  const uint32_t k = a.k, kb_lo = blockIdx.y * a.bps, nkb = min(a.bps, k / 64u - kb_lo);
  const uint32_t pitch = k >> 1;
  constexpr uint32_t kSB = FMT == kINT4 ? 2u : 4u;
  const uint32_t spitch = (k / (is_g128(FMT) ? 128u : 64u)) * kSB;
  // scale bytes before block kb_lo (an even block for the formats with 128-weight groups)
  const uint32_t soff = FMT == kINT4 ? kb_lo : FMT == kINT4A ? kb_lo * 2u : kb_lo * 4u;
  const uint32_t wrow0 = tn * TN + (uint32_t)wave * 32u * NT;
  const uint32_t wbase = wrow0 < mm.n ? wrow0 : 0u;
  const uint32_t wrows = wrow0 < mm.n ? min(32u * NT, mm.n - wrow0) : 0u;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(mm.packed + (size_t)wbase * pitch + kb_lo * 32u,
                                              wrows ? wrows * pitch - kb_lo * 32u : 0u);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(reinterpret_cast<const char*>(mm.scales) + (size_t)wbase * spitch + soff,
                wrows ? wrows * spitch - soff : 0u);
  const uint32_t xrows = min((uint32_t)TM, a.m - m0);
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(a.x + (size_t)m0 * k + kb_lo * 64u, xrows * k * 2u - kb_lo * 128u);
  float* const yz = mm.y + (size_t)blockIdx.y * a.ysplit;

  // Block kb's packed bytes for this lane: row 32 t + c, bytes [16 h, 16 h + 16) of the block;
  // blocks past K and rows past N read as zero.
  uint4 W[DP][NT];
  auto load_w = [&](uint32_t kb, uint4 (&w)[NT]) __attribute__((always_inline)) {
    const bool have = kb < nkb;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t row = (uint32_t)(32 * t + c);
      w[t] = buffer_load16_stream(rw, offset_or_oob(have, row * pitch + kb * 32u + 16u * (uint32_t)h));
    }
  };
  // The scales of blocks 4 q .. 4 q + 3 of this lane's rows in one load per row: four fp32 words
  // (NF4, FP4; 16 bytes at a 4-byte aligned offset) or two bf16 group scales (INT4).
  // One load per row per four blocks instead of one per block (two for INT4): each such load
  // touches one cache line per row, whatever its width.  Words past the row's scales read the next row's (or zero
  // past the wave's rows), which only ever meets blocks past K, whose weights are zero.
  uint4 SQ[2][NT];
  auto load_sq = [&](uint32_t q, uint4 (&sq)[NT]) __attribute__((always_inline)) {
    const bool have = 4u * q < nkb;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t row = (uint32_t)(32 * t + c);
      if constexpr (FMT == kINT4) {
        const uint32_t off = offset_or_oob(have, row * spitch + q * 4u);  // 2-byte aligned
        const uint32_t g0 = buffer_load16bit(rs, off) << 16, g1 = buffer_load16bit(rs, off + 2u) << 16;
        sq[t] = make_uint4(g0, g0, g1, g1);
      } else if constexpr (FMT == kINT4A) {
        // the two groups' words, kept whole (scale and zero point)
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(
            rs, (int)offset_or_oob(have, row * spitch + q * 8u), 0, 0);
        sq[t] = make_uint4(v.x, v.x, v.y, v.y);
      } else {
        sq[t] = buffer_load16(rs, offset_or_oob(have, row * spitch + q * 16u));
      }
    }
  };
  // Stage of block kb into buffer b (every thread moves SLOTS / 256 slots).
  auto load_x = [&](uint32_t kb, int b) __attribute__((always_inline)) {
    const bool have = kb < nkb;
#pragma unroll
    for (int j = 0; j < SLOTS / kFoldThreads; ++j) {
      const uint32_t sl = (uint32_t)(j * kFoldThreads + tid);
      const uint32_t mr = sl >> 3, cc = (sl & 7u) ^ xkey(mr);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)((b ? xs1 : xs0) + j * kFoldThreads + wave * 64), 16,
          (int)offset_or_oob(have, (mr * k + kb * 64u + cc * 8u) * 2u), 0, 0, 0);
    }
  };

#pragma unroll
  for (int i = 0; i < ST - 1; ++i) load_x((uint32_t)i, i);
  load_sq(0, SQ[0]);
#pragma unroll
  for (int i = 0; i < DP; ++i) load_w((uint32_t)i, W[i]);
  if constexpr (FMT != kFP4) fill_table<FMT, kF16, kFoldThreads>(tab);

  f32x16 acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][j][e] = 0.f;

  const uint32_t laneoff = (uint32_t)c * 8u;  // this lane's table copy
  const char* tabc = reinterpret_cast<const char*>(tab);
  auto afrag = [&](int b, int j, int q) __attribute__((always_inline)) {
    const uint32_t mr = (uint32_t)(32 * j + c), cc = (uint32_t)(4 * h + q);
    return (b ? xs1 : xs0)[mr * 8u + (cc ^ xkey(mr))];
  };

  // Block kb of the folded route: the barrier completes stage b (every wave's copies) and ends
  // the reads of the stage the next copy overwrites; then that copy, the decode with the scale
  // folded in, the weight refill DP blocks ahead, the matrix steps.
  auto step = [&](uint32_t kb, int b, uint4 (&w)[NT], const uint32_t (&s)[NT]) __attribute__((always_inline)) {
    wait_own_stage_copies((b ? xs1 : xs0) + tid);
    __syncthreads();
    load_x(kb + ST - 1, (b + ST - 1) % ST);
    uint4 bw[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // s[t]: fp32 bits (NF4, FP4, INT4), the group's word (asymmetric INT4)
      const _Float16 sh = (_Float16)(FMT == kINT4A ? scale_f32<FMT>(s[t]) : __uint_as_float(s[t]));
      const half2_t s2 = {sh, sh};
      const half2_t zz = __builtin_bit_cast(half2_t, FMT == kINT4A ? zero_shift_pair(s[t]) : 0u);
      const uint32_t wd[4] = {w[t].x, w[t].y, w[t].z, w[t].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t p[4];
        decode4<FMT>(wd[q], tabc, laneoff, p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          half2_t v = __builtin_bit_cast(half2_t, p[e]);
          if constexpr (FMT == kINT4A) v = v + zz;  // q - z, exact
          p[e] = __builtin_bit_cast(uint32_t, v * s2);
        }
        bw[t][q] = make_uint4(p[0], p[1], p[2], p[3]);
      }
    }
    load_w(kb + DP, w);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const uint4 af = afrag(b, j, q);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t][j] = mfma32(af, bw[t][q], acc[t][j]);
      }
    }
  };

  // Every block scale of this wave's rows over its K range, checked once: lane (h, c) reads
  // scales h, h + 2, ... of row 32 t + c, one load per scale (rows past N read as zero, which
  // folds).  The loads go out after the first weights and stages, so the check adds no round trip
  // before the first block.
  bool fold = true;
  {
    const uint32_t nsc = is_g128(FMT) ? nkb / 2u : nkb;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t row = (uint32_t)(32 * t + c);
      for (uint32_t i = (uint32_t)h; i < nsc; i += 2u) {
        const uint32_t raw = FMT == kINT4 ? buffer_load16bit(rs, row * spitch + i * 2u)
                                          : buffer_load32(rs, row * spitch + i * 4u);  // INT4A: word
        fold = fold && foldable<FMT>(scale_f32<FMT>(raw));
      }
    }
  }
  const bool fold_wave = __builtin_amdgcn_ballot_w64(!fold) == 0;

  if (fold_wave) {
    // Eight blocks per trip: two scale quads alternate, and stages and weight sets rotate with it.
    constexpr int UNR = 8;
    static_assert(UNR % DP == 0 && UNR % ST == 0, "register sets and stages rotate together");
    auto unit = [&](uint32_t kb0, int u) __attribute__((always_inline)) {
      const uint32_t kb = kb0 + (uint32_t)u;
      uint4 (&sq)[NT] = SQ[(u >> 2) & 1];
      if ((u & 3) == 0) load_sq(kb / 4u + 1u, SQ[((u >> 2) + 1) & 1]);
      uint32_t sw[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        sw[t] = (u & 3) == 0 ? sq[t].x : (u & 3) == 1 ? sq[t].y : (u & 3) == 2 ? sq[t].z : sq[t].w;
      step(kb, u % ST, W[u % DP], sw);  // kb0 is a multiple of UNR, hence of ST
    };
    uint32_t kb = 0;
    for (; kb + UNR <= nkb; kb += UNR) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) unit(kb, u);
    }
#pragma unroll
    for (int u = 0; u < UNR - 1; ++u) {
      if (kb + u < nkb) unit(kb, u);
    }
  } else {
    // every wave runs the same number of barriers on either route
    fold_block_scale_wave<FMT, NT, MT>(rw, rs, rx, reinterpret_cast<const char*>(tab), xs0, xs1, yz,
                                   mm.n, a.m, m0, wrow0, k, nkb);
    return;
  }

  // y[m0 + 32 j + 8 (e / 4) + 4 h + e % 4][wrow0 + 32 t + c]: for each register, 32 lanes write
  // 32 consecutive floats of one row of y.
  const uint32_t n = mm.n;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint32_t col = wrow0 + 32u * t + (uint32_t)c;
    if (col >= n) continue;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t mr = m0 + 32u * j + 8u * (uint32_t)(e >> 2) + 4u * (uint32_t)h + (uint32_t)(e & 3);
        if (mr < a.m) yz[(size_t)mr * n + col] = acc[t][j][e];
      }
    }
  }
}

template <int FMT, int NT, int MT, bool GROUPED>
hipError_t launch_nt(const FoldArgs& a, int ranges, hipStream_t s) {
  // Two activation stages and four blocks of weights in flight (eight blocks per unrolled trip,
  // two quads of scales): measured on MI355X against three stages and three blocks.  Asymmetric
  // INT4 with 128-row tiles keeps two (its zero-point pairs would otherwise spill).
  constexpr int ST = 2, DP = FMT == kINT4A && NT == 1 ? 2 : 4;
  hipLaunchKernelGGL((fold_kernel<FMT, NT, MT, ST, DP, GROUPED>), dim3(a.tiles, ranges),
                     dim3(kFoldThreads), 0, s, a);
  return hipGetLastError();
}

template <int FMT, int MT>
hipError_t launch_mt(const FoldArgs& a, int nt, int ranges, hipStream_t s) {
  if (nt == 2)
    return a.groups > 1 ? launch_nt<FMT, 2, MT, true>(a, ranges, s)
                        : launch_nt<FMT, 2, MT, false>(a, ranges, s);
  return a.groups > 1 ? launch_nt<FMT, 1, MT, true>(a, ranges, s)
                      : launch_nt<FMT, 1, MT, false>(a, ranges, s);
}

// Full 128-row tiles [tile_base, tile_base + count), or (thin) the same tiles as four 32-row
// slices each, or (wide: 128-weight-row tiles only) 192-row tiles.
template <int FMT>
hipError_t launch_fmt(FoldArgs a, int nt, int ranges, int64_t tile_base, int64_t count, bool thin,
                      bool wide, hipStream_t s) {
  a.tile_base = (uint32_t)tile_base;
  a.tiles = (uint32_t)(thin ? count * kFoldMT : count);
  if (wide)
    return a.groups > 1 ? launch_nt<FMT, 1, kWideMT, true>(a, ranges, s)
                        : launch_nt<FMT, 1, kWideMT, false>(a, ranges, s);
  return thin ? launch_mt<FMT, 1>(a, nt, ranges, s) : launch_mt<FMT, kFoldMT>(a, nt, ranges, s);
}

int64_t fold_tiles(const int64_t* ns, int groups, int64_t m, int64_t tn) {
  int64_t t = 0;
  for (int g = 0; g < groups; ++g) t += (ns[g] + tn - 1) / tn;
  return t * ((m + 32 * kFoldMT - 1) / (32 * kFoldMT));
}

}  // namespace

// K ranges of the folded kernel when `splits` are requested over K: blocks per range as for the
// block-scale kernel (ceil(blocks / splits)), rounded up to an even count for INT4 (a range then
// starts on a 128-weight group), so never more ranges than that kernel's.
int gemm_fold_ranges(int fmt, int64_t k, int splits, int64_t* bps) {
  const int64_t nb = k / 64;
  const int64_t sp = std::max<int64_t>(1, std::min<int64_t>(splits, nb));
  int64_t per = (nb + sp - 1) / sp;
  if (fmt == W4_INT4_X_F16 || fmt == W4_INT4A_X_F16) per += per & 1;
  if (bps) *bps = per;
  return (int)((nb + per - 1) / per);
}

bool gemm_fold_format(int fmt) {
  return fmt == W4_NF4_X_F16 || fmt == W4_INT4_X_F16 || fmt == W4_FP4_X_F16 ||
         fmt == W4_INT4A_X_F16;
}

// Weight rows per tile of the folded kernel for an unsplit launch (256 or 128), or 0 when the
// block-scale kernel is the faster one.  Measured on MI355X (rotated weights, against the
// block-scale kernel's automatic launch): at 512 activation rows, 256-row tiles where they number
// two per CU (one per CU for rows of 4096+ weights): NF4 151936 x 1536 334 against 426 us (INT4 x
// fp16 315), 28672 x 8192 289 against 402; else 128-row tiles from one per CU: 8960 x 1536 35
// against 45 us, 8192 x 8192 106 against 129, 8192 x 28672 363 against 423 (the two gate/up
// matrices of a grouped launch: the same as the block-scale kernel's 64 x 128 tiles).  From 128
// activation rows: at 192 rows 151936 x 1536 181 against 208 us, 28672 x 8192 172 against 221,
// 8960 x 1536 22.2 against 31.0; at 128 rows 151936 x 1536 115 against 127 (128-row tiles), while
// 8960 x 1536 (70 tiles) stays with the block-scale kernel (22.5 against 17.3).  With one
// 128-row activation tile (M <= 128) the 256-row tiles lose (151936 x 1536 at 128 rows 127 us
// against 115 with 128-row tiles); from two, 128-row tiles already win at half a tile per CU on
// rows shorter than 4096 weights (8960 x 1536 at 192 rows, 140 tiles: 22.2 us against the
// block-scale kernel's 31.0), not on longer ones, whose few workgroups then carry hundreds of
// blocks each (8192 x 8192 at 192 rows, 128 tiles: 95 against 62.5; 8192 x 28672 352 against
// 207: split over K, the folded kernel wins again).  From 129 to 192 rows a matrix with at least
// one 128-weight-row tile per CU takes 128-row tiles, which the launch runs as 192-row activation
// tiles: ahead of the 256-row ones (192 rows: 151936 x 1536 131 us against 169, 128256 x 8192
// 524 against 720).
int gemm_fold_tile_rows(int fmt, const int64_t* ns, int groups, int64_t k, int64_t m) {
  if (!gemm_fold_format(fmt) || m < 128 || k < 64 || k % 64 != 0) return 0;
  const int64_t cus = device_cu_count();
  // 129 to 192 rows: 192-row tiles over 128 weight rows wherever they give every CU one
  if (m > 128 && m <= 32 * kWideMT && 32 * kWideMT * k * 2 < ((int64_t)1 << 31) &&
      fold_tiles(ns, groups, 1, 128) >= cus)
    return 128;
  if (m > 128 && fold_tiles(ns, groups, m, 256) >= (k >= 4096 ? cus : 2 * cus)) return 256;
  const int64_t t128 = fold_tiles(ns, groups, m, 128);
  if (t128 >= cus || (m > 128 && k < 4096 && 2 * t128 >= cus)) return 128;
  return 0;
}

// K ranges the automatic tiled path gives the folded kernel (128-row tiles) on one matrix, 1 for
// none, or 0 where the kernel does not apply (below 256 activation rows, fewer than 32 tiles:
// the block-scale kernel's split is faster there).  With T tiles below one per CU and rows of
// 4096+ weights: S = min(16, 2 CUs / T) (about two workgroups per CU) when that leaves 32+ blocks
// per range, else S = min(16, CUs / T, K / 64 / 12) (at least 12 blocks each), at least 2 from
// half a tile per CU, when that is 2 or more; from one to two tiles per CU with rows of 16384+
// weights: two ranges (two workgroups per CU).  Long rows gain from the second workgroup per CU
// (8192 x 8192 at 192 rows: 57.5 us over four ranges against 61.9 over two; 8192 x 28672 at 128
// rows 112 over eight against 118 over four, at 192 rows 183 over four against 194 over two),
// short ones do not (1536 x 8960 at 512 rows over ten ranges 36.9 against 36.7 over five).  Measured on MI355X (NF4 x fp16, rotated weights; INT4 within 5%): 1536 x
// 8960 at 512 activation rows (48 tiles) 120 us unsplit, 67.8 / 50.1 / 41.6 / 36.7 / 40.3 / 39.8 /
// 36.9 at S = 2 / 3 / 4 / 5 / 6 / 8 / 10 (the block-scale kernel's split: 44.4); at 256 rows (24
// tiles) 38.6 / 32.7 / 26.9 / 24.3 / 28.2 at S = 4 / 5 / 8 / 10 / 16 (27.4); 1024 x 8192 at 512
// (32 tiles) 34.7 / 28.1 / 26.1 / 29.3 at S = 4 / 6 / 8 / 10 (25.5); 8192 x 28672 at 512 (256
// tiles) 363 / 339 / 354 at S = 1 / 2 / 3; 8192 x 8192 at 512 106 / 105 at S = 1 / 2 (not
// split); 1536 x 1536 at 512 (24 blocks) 18.5 at best, against the MFMA path's 12.4 (not split).
// At 128 activation rows: 28672 x 8192 (224 tiles) 112 us over two ranges against 119 unsplit and
// the block-scale kernel's 127; 8192 x 28672 (64 tiles) 118 / 112 over four / eight against 131;
// 8192 x 8192 (64) 42.0 over four against 42.5; 1536 x 8960 (12 tiles) 25.7 over eight against the
// block-scale kernel's 21.4 (hence its share below 32 tiles).
int gemm_fold_auto_splits(int fmt, int64_t n, int64_t k, int64_t m) {
  if (!gemm_fold_format(fmt) || m < 128 || k < 64 || k % 64 != 0) return 0;
  const int64_t cus = device_cu_count();
  const int64_t nb = k / 64;
  const int64_t tiles = fold_tiles(&n, 1, m, 128);
  if (m < 256 && tiles < 32) return 0;
  if (tiles < cus) {
    if (nb < 64) return 1;
    // about two workgroups per CU while the ranges keep 32+ blocks, else about one
    const int64_t s2 = std::min<int64_t>(16, 2 * cus / tiles);
    if (s2 >= 2 && nb / s2 >= 32) return (int)s2;
    int64_t s = std::min<int64_t>(std::min<int64_t>(16, cus / tiles), nb / 12);
    if (2 * tiles >= cus) s = std::max<int64_t>(s, std::min<int64_t>(2, nb / 12));
    return s >= 2 ? (int)s : 1;
  }
  return tiles < 2 * cus && nb >= 256 ? 2 : 1;
}

// Split tiled launches (one member) of the formats and sizes the folded kernel runs: from 256
// activation rows, and from 128 with at least 32 tiles of 128 rows (the split rule above).
bool gemm_fold_split(int fmt, int groups, const int64_t* ns, int64_t m) {
  return gemm_fold_format(fmt) && groups == 1 &&
         (m >= 256 || (m >= 128 && fold_tiles(ns, 1, m, 128) >= 32));
}

hipError_t launch_gemm_fold(int fmt, const uint16_t* x, int groups, const uint8_t* const* packed,
                            const void* const* scales, const int64_t* ns, float* const* y,
                            int64_t k, int64_t m, int tile_rows, hipStream_t s, int splits,
                            float* ws) {
  if (!gemm_fold_format(fmt) || groups < 1 || groups > kMaxGroup || m < 1 || k < 64 || k % 64 != 0)
    return hipErrorInvalidValue;
  if ((fmt == W4_INT4_X_F16 || fmt == W4_INT4A_X_F16) && k % 128 != 0) return hipErrorInvalidValue;
  if (tile_rows != 128 && tile_rows != 256) return hipErrorInvalidValue;
  int64_t n_total = 0;
  for (int g = 0; g < groups; ++g) {
    if (ns[g] < 1) return hipErrorInvalidValue;
    n_total += ns[g];
  }
  // 32-bit offsets inside the buffer resources: 128 activation rows and 64 weight rows of K.
  if (128 * k * 2 >= ((int64_t)1 << 31) || n_total >= ((int64_t)1 << 31) || m >= ((int64_t)1 << 31))
    return hipErrorNotSupported;
  int64_t bps = 0;
  const int ranges = gemm_fold_ranges(fmt, k, splits, &bps);
  if (ranges > 1 && (groups > 1 || !ws)) return hipErrorInvalidValue;
  if (ranges > 1 && m * ns[0] >= ((int64_t)1 << 32)) return hipErrorNotSupported;  // 32-bit planes
  // 129 to 192 activation rows in one 192-row tile instead of two 128-row ones (the second a
  // half padding), for unsplit 128-weight-row tiles that still give every CU one tile: each
  // weight is then decoded once, and a quarter fewer matrix steps run.
  const int64_t cus = device_cu_count();
  const bool wide = ranges == 1 && tile_rows == 128 && m > 128 && m <= 32 * kWideMT &&
                    32 * kWideMT * k * 2 < ((int64_t)1 << 31) && fold_tiles(ns, groups, 1, 128) >= cus;
  const int64_t mt = wide ? 1 : (m + 32 * kFoldMT - 1) / (32 * kFoldMT);
  const int64_t tiles = wide ? fold_tiles(ns, groups, 1, 128) : fold_tiles(ns, groups, m, tile_rows);
  if (tiles >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  FoldArgs a;
  int64_t tile0 = 0;
  for (int g = 0; g < kMaxGroup; ++g) {
    const bool use = g < groups;
    a.mb[g].packed = use ? packed[g] : packed[0];
    a.mb[g].scales = use ? scales[g] : scales[0];
    a.mb[g].y = use ? (ranges > 1 ? ws : y[g]) : nullptr;
    a.mb[g].n = use ? (uint32_t)ns[g] : 0u;
    a.mb[g].tile0 = use ? (uint32_t)tile0 : 0xFFFFFFFFu;
    if (use) tile0 += ((ns[g] + tile_rows - 1) / tile_rows) * mt;
  }
  a.x = x;
  a.groups = (uint32_t)groups;
  a.m = (uint32_t)m;
  a.k = (uint32_t)k;
  a.mt = (uint32_t)mt;
  a.bps = (uint32_t)bps;
  a.ysplit = ranges > 1 ? (uint32_t)(m * ns[0]) : 0u;
  const int nt = tile_rows / 128;
  // Two workgroups per CU hold 2 * CUs tiles at once.  One pass whose tiles leave a last round of
  // at most CUs / 4 tiles (whole rounds before it) runs that round as a second launch of 32-row
  // slices, four per tile, spread over the CUs: the sums over K take the same order either way.
  const int64_t slots = 2 * cus, rem = tiles % slots;
  const int64_t tail = !wide && ranges == 1 && tiles > slots && 4 * rem <= slots / 2 ? rem : 0;
  auto run = [&](int64_t base, int64_t count, bool thin) {
    switch (fmt) {
      case W4_NF4_X_F16: return launch_fmt<kNF4>(a, nt, ranges, base, count, thin, wide, s);
      case W4_INT4_X_F16: return launch_fmt<kINT4>(a, nt, ranges, base, count, thin, wide, s);
      case W4_INT4A_X_F16: return launch_fmt<kINT4A>(a, nt, ranges, base, count, thin, wide, s);
      case W4_FP4_X_F16: return launch_fmt<kFP4>(a, nt, ranges, base, count, thin, wide, s);
    }
    return hipErrorInvalidValue;
  };
  hipError_t e = run(0, tiles - tail, false);
  if (e == hipSuccess && tail > 0) e = run(tiles - tail, tail, true);
  if (e != hipSuccess || ranges == 1) return e;
  // the ranges' partial sums, added in range order into y
  return launch_splitk_reduce(ws, y[0], m * ns[0], ranges, s);
}

}  // namespace w4
