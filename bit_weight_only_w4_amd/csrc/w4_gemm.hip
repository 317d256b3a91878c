// Prefill-size GEMM: y[m, n] = sum_k x[m, k] * W_hat[n, k] for hundreds to thousands of activation
// rows (the tokens of a prompt), the weights decoded on chip and multiplied on the matrix cores.
//
// A GEMV kernel run once per token makes prefill an order of magnitude slower than a GEMM (LLM
// Quantization on RTX 4060, "Why Only 16%", item 3); the dequantize-then-dense-GEMM route rebuilds
// the fp16 matrix on every call (Do Quantization and Sparsity make LLM Inference Faster?, "NF4:
// fast at batch 1, slower at larger batches").  Here each workgroup owns an output tile of
// TN weight rows x TM activation rows and walks K one 64-weight block at a time, so every decoded
// weight is reused by TM activation rows and every activation by TN weight rows: the work is
// bound by the matrix cores, not by memory.
//
// Work layout.  A K group is 256 threads = 4 waves in a 2 x 2 grid over the tile; wave (wn, wm)
// owns WN row tiles x WM column tiles of 16 x 16 outputs (TN = 32 WN, TM = 32 WM).  A workgroup has
// KW K groups that split the K blocks between them and add their sums through LDS at the end in a
// fixed order (small grids: twice the waves per tile and half the blocks per wave).
//   * A operand (16 weight rows x 32 k per MFMA step): lane l = 16 g + r takes row r and the 8
//     consecutive weights 16 g + 8 s .. 16 g + 8 s + 7 of the block in step s = 0, 1: bytes
//     [8 g, 8 g + 8) of the row's 32-byte block, one 8-byte load per row tile, decoded pairwise
//     through the byte -> pair table in LDS.  Both steps lie inside one scale block, so the block
//     scale is applied exactly, in fp32, to the block's fresh partial sums: acc += scale * D.
//     INT4 groups of 128 are two such blocks under one scale.  Asymmetric INT4 decodes q - 8 as
//     INT4 and adds one MFMA per step whose A rows hold -(z - 8): D becomes the sum of (q - z) x.
//   * B operand (32 k x 16 activation rows): lane l = 16 g + r takes activation row r of the
//     column tile and the same 8 k positions, one ds_read_b128 from the x stage in LDS.
//   * x stages: the tile's TM activation rows x 64 k (128 bytes per row, padded to 144 so that
//     the 16 lanes of a read hit distinct banks), double-buffered in LDS per K group.  Stage kb + 2 is
//     loaded into registers when block kb starts (two register sets) and written to LDS at the
//     end of block kb + 1; one barrier per block.
//   * Weights and scales run four blocks ahead of the multiply (four register sets, rotating by
//     unrolling): a block's loads have three blocks of matrix work to land.
//   * D (16 x 16 fp32): lane l = 16 g + r holds weight rows 4 g .. 4 g + 3 of activation row r,
//     consecutive in y[m, :] (one 16-byte store).
//   * Workgroups are numbered so that the ones the dispatcher places on one XCD (every eighth)
//     take consecutive tiles, the activation-row tiles of one weight-row tile first: a weight tile
//     is read from HBM once and then served by that XCD's L2.
#include <algorithm>

#include "w4_mfma_common.h"

namespace w4 {

// One matrix of a launch.  The matrices of a grouped launch share x and K; their tiles are
// numbered one after another, member g owning tiles [tile0, tile0 + mt * its weight-row tiles).
struct GemmMember {
  const uint8_t* packed;  // [N_g, K/2]
  const void* scales;     // NF4, FP4 float[N_g, K/64] | INT4 uint16 / INT4A uint32 [N_g, K/128]
  float* y;               // [M, N_g], or the partial sums [S, M, N] of a split K (one member)
  uint32_t n;             // N_g
  uint32_t tile0;
};

struct GemmArgs {
  GemmMember mb[kMaxGroup];
  const uint16_t* x;      // [M, K] activations (bits)
  uint32_t groups;
  uint32_t m, k;
  uint32_t mt;            // activation-row tiles (TM rows each)
  uint32_t tiles;         // tiles of all members
  uint32_t bps;           // 64-weight blocks per K range: range z = blockIdx.y owns blocks
                          // [z bps, min((z + 1) bps, K / 64)) and writes y + z * ysplit
  uint32_t ysplit;        // floats between the partial planes of consecutive ranges (M * N)
};

namespace {

constexpr int kGroupThreads = 256;            // one K group: 4 waves in a 2 x 2 grid
constexpr int kXPitch = 144;                  // LDS bytes per activation row of a stage
constexpr int kXcds = 8;
constexpr int kDepth = 4;                     // weight blocks in flight (register sets)

template <int WM>
constexpr int stage_bytes() { return 32 * WM * kXPitch; }

// Weights and scales of one block for this lane: two dwords of packed bytes per row tile, and the
// scale of D row 4 g + (r & 3) of each row tile (fp32 bits; INT4: bf16 bits in the low half).
template <int WN>
struct Block {
  uint32_t w[WN][2];
  uint32_t s[WN];
};

template <int FMT, int XT, int WN, int WM, int KW, bool GROUPED>
__global__ void __launch_bounds__(kGroupThreads * KW, 2) gemm_kernel(GemmArgs a) {
  constexpr int TN = 32 * WN, TM = 32 * WM;
  constexpr bool kSplit = FMT == kNF4 && XT == kBF16;
  constexpr int SB = FMT == kINT4 ? 2 : 4;  // bytes per scale (INT4A: its 32-bit word)
  // LDS: the decode table (static, at address 0, so a lookup address needs no base), then the two
  // x stages of each K group (dynamic), reused at the end for the K groups' sums.
  __shared__ __align__(16) uint32_t tab[kTableBytes / 4];
  extern __shared__ __align__(16) uint8_t xs[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wm = (wave >> 1) & 1, kg = wave >> 2;
  const int gt = tid & (kGroupThreads - 1);  // thread index inside the K group
  const int g = lane >> 4, r = lane & 15;

  // This workgroup's tile: every eighth workgroup shares an XCD; those take consecutive tiles.
  const uint32_t id = blockIdx.x, tiles = a.tiles;
  const uint32_t xcd = id % kXcds, per = tiles / kXcds, extra = tiles % kXcds;
  const uint32_t tile = xcd * per + min(xcd, extra) + id / kXcds;
  // Its member, by selects over the fixed member slots (the argument block is never indexed by a
  // computed value).
  GemmMember mm = a.mb[0];
  if constexpr (GROUPED) {
#pragma unroll
    for (int i = 1; i < kMaxGroup; ++i) {
      if ((uint32_t)i < a.groups && tile >= a.mb[i].tile0) mm = a.mb[i];
    }
  }
  const uint32_t lt = tile - mm.tile0;
  const uint32_t tn = lt / a.mt, tm = lt - tn * a.mt;
  const uint32_t n0 = tn * TN, m0 = tm * TM;

  const uint32_t k = a.k;
  // This workgroup's K range: blocks [kb0, kb0 + nbz) of 64 weights (all of K without a split;
  // the host makes every range non-empty).
  const uint32_t kb0 = blockIdx.y * a.bps;
  const uint32_t nbz = min(a.bps, k / 64u - kb0);
  // K group kg takes blocks [kbase, kbase + cnt); every group runs `steps` block steps (the
  // barriers are shared), the ones past its range on zero-filled loads, which add nothing.
  const uint32_t steps = (nbz + KW - 1) / KW;
  const uint32_t kfirst = (uint32_t)kg * steps;
  const uint32_t kbase = kb0 + kfirst;
  const uint32_t cnt = kfirst < nbz ? min(steps, nbz - kfirst) : 0u;
  const uint32_t pitch = k >> 1;     // packed bytes per weight row
  const uint32_t spitch = (k / (is_g128(FMT) ? 128 : 64)) * SB;

  // Buffer resources: this wave's WN * 16 weight rows (rows past N read as zero), and the
  // workgroup's TM activation rows (rows past M read as zero).
  const uint32_t wrow0 = n0 + (uint32_t)wn * 16u * WN;
  const uint32_t wrows = wrow0 < mm.n ? min(16u * WN, mm.n - wrow0) : 0u;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(mm.packed + (size_t)wrow0 * pitch, wrows * pitch);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(reinterpret_cast<const char*>(mm.scales) + (size_t)wrow0 * spitch, wrows * spitch);
  const uint32_t xrows = min((uint32_t)TM, a.m - m0);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x + (size_t)m0 * k, xrows * k * 2u);

  // Per-lane offsets: packed bytes of row r, lane group g; the scale row 4 g + (r & 3).
  const uint32_t woff = (uint32_t)r * pitch + 8u * (uint32_t)g;
  const uint32_t soff = (uint32_t)(4 * g + (r & 3)) * spitch;

  auto load_block = [&](uint32_t i, Block<WN>& d) __attribute__((always_inline)) {
    const bool have = i < cnt;
    const uint32_t kb = kbase + i;
#pragma unroll
    for (int t = 0; t < WN; ++t) {
      const uint32_t off = offset_or_oob(have, woff + (uint32_t)t * 16u * pitch + kb * 32u);
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)off, 0, 0);
      d.w[t][0] = v.x;
      d.w[t][1] = v.y;
    }
    if constexpr (is_g128(FMT)) {
#pragma unroll
      for (int t = 0; t < WN; ++t) {
        const uint32_t row = soff + (uint32_t)t * 16u * spitch;
        if constexpr (FMT == kINT4A) {
          d.s[t] = buffer_load32(rs, offset_or_oob(have, row + (kb >> 1) * 4u));
        } else {
          d.s[t] = buffer_load16bit(rs, offset_or_oob(have, row + (kb >> 1) * 2u));
        }
      }
    }
  };
  // NF4 and FP4: the fp32 scales of QS consecutive blocks i .. i + QS - 1 (of this K group) in one
  // load per row tile every QS blocks (four blocks, 16 bytes; two, 8 bytes, with 128 x 128 tiles,
  // whose registers hold no more).  A dword per block touched one cache line per row for 4 useful
  // bytes; words past the group's blocks belong to later blocks or the next row (or read zero past
  // the rows), and only ever meet blocks past the range, whose weights read as zero.
  constexpr int QS = WN >= 4 ? 2 : 4;
  auto load_sq = [&](uint32_t i, uint4 (&sq)[WN]) __attribute__((always_inline)) {
    const bool have = i < cnt;
#pragma unroll
    for (int t = 0; t < WN; ++t) {
      const uint32_t row = soff + (uint32_t)t * 16u * spitch;
      const uint32_t off = offset_or_oob(have, row + (kbase + i) * 4u);
      if constexpr (QS == 4) {
        sq[t] = buffer_load16(rs, off);
      } else {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)off, 0, 0);
        sq[t] = make_uint4(v.x, v.y, 0u, 0u);
      }
    }
  };
  // x stage of the group's block i: group thread gt moves 16-byte chunks c = gt + 256 j (row
  // c / 8, chunk c % 8) into the group's own two stages.
  uint8_t* xg = xs + (uint32_t)kg * 2u * stage_bytes<WM>();
  auto load_x = [&](uint32_t i, uint4 (&xr)[WM]) __attribute__((always_inline)) {
    const uint32_t kb = kbase + i;
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      const uint32_t c = (uint32_t)gt + (uint32_t)kGroupThreads * j;
      const uint32_t row = c >> 3, col = c & 7u;
      xr[j] = buffer_load16(rx, offset_or_oob(i < cnt, row * k * 2u + kb * 128u + col * 16u));
    }
  };
  auto store_x = [&](int buf, const uint4 (&xr)[WM]) __attribute__((always_inline)) {
    uint8_t* st = xg + buf * stage_bytes<WM>();
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      const uint32_t c = (uint32_t)gt + (uint32_t)kGroupThreads * j;
      *reinterpret_cast<uint4*>(st + (c >> 3) * kXPitch + (c & 7u) * 16u) = xr[j];
    }
  };

  // Prologue.  Weights run kDepth blocks ahead of the multiply (kDepth register sets), activations
  // two stages ahead (two register sets feeding the two LDS stages).  The loads go out in the
  // loop's steady-state order (weights of blocks 0 .. kDepth - 2, stage 1, weights of block
  // kDepth - 1), so that the waits the compiler derives for the loop entry match its back edge.
  Block<WN> D[kDepth];
  uint4 X0[WM], X1[WM];
  uint4 SQ[2][WN];  // NF4, FP4: scale sets of QS blocks (load_sq), alternating
  if constexpr (!is_g128(FMT)) load_sq(0, SQ[0]);
#pragma unroll
  for (int i = 0; i < kDepth - 1; ++i) load_block((uint32_t)i, D[i]);
  load_x(0, X0);
  fill_table<FMT, XT, kGroupThreads * KW>(tab);
  store_x(0, X0);
  __builtin_amdgcn_sched_barrier(0);
  load_x(1, X1);
  __builtin_amdgcn_sched_barrier(0);
  load_block(kDepth - 1, D[kDepth - 1]);
  __syncthreads();

  float4_t acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i) {
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Twice this lane's byte offset in a table entry (see the lookup below).
  const uint32_t laneoff = kSplit ? (uint32_t)(lane & 15) * 16u : (uint32_t)(lane & 31) * 8u;
  const char* tabc = reinterpret_cast<const char*>(tab);
  // This lane's B fragment offset inside a stage: activation row wm * 16 WM + r, bytes 32 g.
  const uint32_t xoff = ((uint32_t)wm * 16u * WM + (uint32_t)r) * kXPitch + 32u * (uint32_t)g;

  auto compute = [&](int buf, const Block<WN>& d, const uint32_t (&sw)[WN]) __attribute__((always_inline)) {
    const uint8_t* st = xg + buf * stage_bytes<WM>() + xoff;
    uint4 bf[2][WM];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int j = 0; j < WM; ++j)
        bf[s][j] = *reinterpret_cast<const uint4*>(st + j * 16 * kXPitch + s * 16);
    }
#pragma unroll
    for (int t = 0; t < WN; ++t) {
      float4_t dd[WM];
      // INT4A: A operand whose row r is -(z_r - 8) everywhere (the word of row r sits in lane
      // 16 (r >> 2) + (r & 3)); its product adds -(z - 8) * sum(x) to D: codes q - 8 become q - z.
      uint4 zrow = make_uint4(0u, 0u, 0u, 0u);
      if constexpr (FMT == kINT4A) {
        const uint32_t word = (uint32_t)__shfl((int)d.s[t], 16 * (r >> 2) + (r & 3));
        const float zn = (float)(8 - (int)((word >> 16) & 15u));
        const uint32_t h = XT == kF16 ? f16_bits(zn) : (__float_as_uint(zn) >> 16);
        const uint32_t hh = h | (h << 16);
        zrow = make_uint4(hh, hh, hh, hh);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint32_t p1[4], p2[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          // LDS byte address = byte * 128 + lane offset: the perm builds byte * 256 + 2 * lane
          // offset (the packed byte into byte 1), halved by the shift.
          const uint32_t addr =
              __builtin_amdgcn_perm(d.w[t][s], laneoff, 0x0C0C0000u | ((4u + (uint32_t)kb) << 8)) >> 1;
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
        for (int j = 0; j < WM; ++j) {
          dd[j] = mfma<XT>(a1, bf[s][j], s == 0 ? float4_t{0.f, 0.f, 0.f, 0.f} : dd[j]);
          if (kSplit) dd[j] = mfma<XT>(make_uint4(p2[0], p2[1], p2[2], p2[3]), bf[s][j], dd[j]);
          if (FMT == kINT4A) dd[j] = mfma<XT>(zrow, bf[s][j], dd[j]);
        }
      }
      const uint32_t sraw = !is_g128(FMT) ? sw[t] : d.s[t] << 16;
      const float sc[4] = {row_bcast<0>(sraw), row_bcast<1>(sraw), row_bcast<2>(sraw),
                           row_bcast<3>(sraw)};
#pragma unroll
      for (int j = 0; j < WM; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][j][i] = __builtin_fmaf(dd[j][i], sc[i], acc[t][j][i]);
      }
    }
  };

  // Block kb (stage kb % 2, weights in d): fetch stage kb + 2 into the free register set xn
  // (stage kb went to LDS one block ago), multiply, publish stage kb + 1 (register set xp, loaded
  // one block ago) to the other LDS stage, fetch the weights of block kb + kDepth into d.  The
  // barrier ends the reads of stage kb % 2 and makes stage kb + 1 visible.  The x loads are kept
  // ahead of the weight loads (the scheduler would otherwise mix them, and the wait before the LDS
  // store would then also wait for weights fetched later).
  auto step = [&](uint32_t kb, Block<WN>& d, uint4 (&xn)[WM], const uint4 (&xp)[WM],
                  const uint32_t (&sw)[WN]) __attribute__((always_inline)) {
    load_x(kb + 2, xn);
    __builtin_amdgcn_sched_barrier(0);
    compute((int)(kb & 1u), d, sw);
    store_x((int)((kb + 1) & 1u), xp);
    __builtin_amdgcn_sched_barrier(0);
    load_block(kb + kDepth, d);
    __syncthreads();
  };
  // Block kb = kb0 + u of a trip (kb0 a multiple of its length): register set u % 4, activation
  // stage parity u % 2, scale set (u / QS) % 2, whose successor is requested at u % QS == 0.
  auto unit = [&](uint32_t kb0, int u) __attribute__((always_inline)) {
    const uint32_t kb = kb0 + (uint32_t)u;
    uint32_t sw[WN] = {};
    if constexpr (!is_g128(FMT)) {
      uint4 (&sq)[WN] = SQ[(u / QS) & 1];
      if (u % QS == 0) load_sq(kb + QS, SQ[(u / QS + 1) & 1]);
      const int e = u % QS;
#pragma unroll
      for (int t = 0; t < WN; ++t)
        sw[t] = e == 0 ? sq[t].x : e == 1 ? sq[t].y : e == 2 ? sq[t].z : sq[t].w;
    }
    if (u & 1) {
      step(kb, D[u & 3], X1, X0, sw);
    } else {
      step(kb, D[u & 3], X0, X1, sw);
    }
  };

  uint32_t kb = 0;
  if constexpr (is_g128(FMT)) {
    // Four blocks per trip, the register sets rotating (the scales travel with the weights).
    const uint32_t sw0[WN] = {};
    for (; kb + 4 <= steps; kb += 4) {
      step(kb, D[0], X0, X1, sw0);
      step(kb + 1, D[1], X1, X0, sw0);
      step(kb + 2, D[2], X0, X1, sw0);
      step(kb + 3, D[3], X1, X0, sw0);
    }
    if (kb < steps) step(kb, D[0], X0, X1, sw0);
    if (kb + 1 < steps) step(kb + 1, D[1], X1, X0, sw0);
    if (kb + 2 < steps) step(kb + 2, D[2], X0, X1, sw0);
  } else {
    // Eight blocks per trip: the scale sets alternate as well.
    for (; kb + 8 <= steps; kb += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) unit(kb, u);
    }
#pragma unroll
    for (int u = 0; u < 7; ++u) {
      if (kb + u < steps) unit(kb, u);
    }
  }

  // K groups 1 .. KW - 1 hand their sums to group 0 through LDS (the x stages are free after the
  // last barrier), which adds them in the fixed order kg = 1, 2, ...: bitwise reproducible.
  if constexpr (KW > 1) {
    float4_t* red = reinterpret_cast<float4_t*>(xs);
    const int wg4 = wave & 3;
    if (kg > 0) {
#pragma unroll
      for (int t = 0; t < WN; ++t) {
#pragma unroll
        for (int j = 0; j < WM; ++j)
          red[((((kg - 1) * 4 + wg4) * WN + t) * WM + j) * 64 + lane] = acc[t][j];
      }
    }
    __syncthreads();
    if (kg > 0) return;
    for (int q = 1; q < KW; ++q) {
#pragma unroll
      for (int t = 0; t < WN; ++t) {
#pragma unroll
        for (int j = 0; j < WM; ++j) {
          const float4_t v = red[((((q - 1) * 4 + wg4) * WN + t) * WM + j) * 64 + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][j][i] += v[i];
        }
      }
    }
  }

  // Stores: lane (g, r) holds y[m0 + wm * 16 WM + 16 j + r][wrow0 + 16 t + 4 g + i] (of this K
  // range's plane of partial sums when K is split).
  const uint32_t n = mm.n;
  float* yz = mm.y + (size_t)blockIdx.y * a.ysplit;
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    const uint32_t mrow = m0 + (uint32_t)wm * 16u * WM + 16u * j + (uint32_t)r;
    if (mrow >= a.m) continue;
    float* yr = yz + (size_t)mrow * n;
#pragma unroll
    for (int t = 0; t < WN; ++t) {
      const uint32_t col = wrow0 + 16u * t + 4u * (uint32_t)g;
      if ((n & 3u) == 0 && col + 3 < n) {
        *reinterpret_cast<float4_t*>(yr + col) = acc[t][j];
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (col + i < n) yr[col + i] = acc[t][j][i];
        }
      }
    }
  }
}

template <int FMT, int XT, int WN, int WM, int KW, bool GROUPED>
hipError_t launch_wm(const GemmArgs& a, hipStream_t s) {
  static bool raised = false;
  constexpr int lds = KW * 2 * stage_bytes<WM>();
  static_assert(KW == 1 || (KW - 1) * 4 * WN * WM * 64 * 16 <= lds, "K-group sums fit the stages");
  if (!raised) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_kernel<FMT, XT, WN, WM, KW, GROUPED>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    raised = true;
  }
  hipLaunchKernelGGL((gemm_kernel<FMT, XT, WN, WM, KW, GROUPED>),
                     dim3(a.tiles, (a.k / 64 + a.bps - 1) / a.bps), dim3(kGroupThreads * KW), lds, s, a);
  return hipGetLastError();
}

template <int FMT, int XT, bool GROUPED>
hipError_t launch_plan(const GemmArgs& a, int wn, int wm, int kw, hipStream_t s) {
  if (wn == 2 && wm == 4 && kw == 2) return launch_wm<FMT, XT, 2, 4, 2, GROUPED>(a, s);
  if (wn == 2 && wm == 4 && kw == 1) return launch_wm<FMT, XT, 2, 4, 1, GROUPED>(a, s);
  if (wn == 4 && wm == 4 && kw == 1) return launch_wm<FMT, XT, 4, 4, 1, GROUPED>(a, s);
  return hipErrorInvalidValue;
}

template <int FMT, int XT>
hipError_t launch_fx(const GemmArgs& a, int wn, int wm, int kw, hipStream_t s) {
  return a.groups > 1 ? launch_plan<FMT, XT, true>(a, wn, wm, kw, s)
                      : launch_plan<FMT, XT, false>(a, wn, wm, kw, s);
}

// K ranges of a split over `nb` 64-weight blocks when `splits` are requested: ceil(nb / bps)
// with bps = ceil(nb / splits) blocks each (every range non-empty).
int gemm_ranges(int64_t nb, int splits, int64_t* bps) {
  const int64_t s = std::max<int64_t>(1, std::min<int64_t>(splits, nb));
  const int64_t per = (nb + s - 1) / s;
  if (bps) *bps = per;
  return (int)((nb + per - 1) / per);
}

}  // namespace

int gemm_splits_used(int64_t k, int splits) { return gemm_ranges(k / 64, splits, nullptr); }

hipError_t launch_gemm_members(int fmt, const uint16_t* x, int groups, const uint8_t* const* packed,
                               const void* const* scales, const int64_t* ns, float* const* y,
                               int64_t k, int64_t m, hipStream_t s, int splits, float* ws) {
  if (groups < 1 || groups > kMaxGroup || m < 1 || k < 64 || k % 64 != 0)
    return hipErrorInvalidValue;
  int64_t n_total = 0;
  for (int g = 0; g < groups; ++g) {
    if (ns[g] < 1) return hipErrorInvalidValue;
    n_total += ns[g];
  }
  // 32-bit offsets inside the buffer resources: 128 activation rows and 64 weight rows of K.
  if (128 * k * 2 >= ((int64_t)1 << 31) || n_total >= ((int64_t)1 << 31) || m >= ((int64_t)1 << 31))
    return hipErrorNotSupported;
  int64_t bps = 0;
  const int ranges = gemm_ranges(k / 64, splits, &bps);
  if (ranges > 1 && (groups > 1 || !ws)) return hipErrorInvalidValue;
  if (ranges > 1 && m * ns[0] >= ((int64_t)1 << 32)) return hipErrorNotSupported;  // 32-bit planes
  // fp16 activations: the folded-scale kernel in one pass where its tiles fill the CUs, and over
  // K ranges (128-row tiles) where its split rule takes it
  if (ranges == 1) {
    const int fold_rows = gemm_fold_tile_rows(fmt, ns, groups, k, m);
    if (fold_rows > 0)
      return launch_gemm_fold(fmt, x, groups, packed, scales, ns, y, k, m, fold_rows, s);
  } else if (gemm_fold_split(fmt, groups, ns, m)) {
    return launch_gemm_fold(fmt, x, groups, packed, scales, ns, y, k, m, 128, s, splits, ws);
  }
  const int64_t cus = device_cu_count();
  const int wm = 4;
  const int64_t mt = (m + 32 * wm - 1) / (32 * wm);
  auto tiles_of = [&](int64_t rows) {
    int64_t t = 0;
    for (int g = 0; g < groups; ++g) t += (ns[g] + rows - 1) / rows;
    return t * mt;
  };
  // 128 x 128 tiles (one K group) when there are enough of them, counting every member's and
  // every K range's: 1.5 per CU for rows of at least 4096 weights, 4 per CU for shorter rows;
  // else 64 x 128 tiles, with one K group when those make two workgroups per CU, two K groups
  // (twice the waves per tile, half the blocks per wave) when they do not.  The larger tile halves
  // the activation traffic per weight; the smaller one fills the CUs more evenly, which matters
  // most for short rows (few blocks per tile).  Measured on MI355X (NF4 x fp16, 128 x 128 against
  // 64 x 128 tiles): 16032 x 8192 at 512 activation rows (504 tiles of 128 x 128) 218 against
  // 245 us, 2 x 28672 x 8192 at 256 (448) 429 against 443, 8192 x 8192 at 512 (256) 133 against
  // 129; 2 x 8960 x 1536 at 512 (560) 76.3 against 68.9, at 1024 (1120) 120.8 against 120.1,
  // 151936 x 1536 at 128 (1187) 145 against 151; at 512 activation rows 1536 x 8960 takes 71.9 us
  // with two K groups against 85.5 with one.  Larger tiles (128 x 256 or 256 x 128 per workgroup,
  // one wave per SIMD) measured 1.4-5x slower.
  const bool full = tiles_of(128) * ranges >= (k >= 4096 ? 3 * cus / 2 : 4 * cus);
  const bool half = !full && tiles_of(64) * ranges >= 2 * cus;
  const int wn = full ? 4 : 2, kw = full || half ? 1 : 2;
  const int64_t tiles = tiles_of(32 * wn);
  if (tiles >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  GemmArgs a;
  int64_t tile0 = 0;
  for (int g = 0; g < kMaxGroup; ++g) {
    const bool use = g < groups;
    a.mb[g].packed = use ? packed[g] : packed[0];
    a.mb[g].scales = use ? scales[g] : scales[0];
    a.mb[g].y = use ? (ranges > 1 ? ws : y[g]) : nullptr;
    a.mb[g].n = use ? (uint32_t)ns[g] : 0u;
    a.mb[g].tile0 = use ? (uint32_t)tile0 : 0xFFFFFFFFu;
    if (use) tile0 += ((ns[g] + 32 * wn - 1) / (32 * wn)) * mt;
  }
  a.x = x;
  a.groups = (uint32_t)groups;
  a.m = (uint32_t)m;
  a.k = (uint32_t)k;
  a.mt = (uint32_t)mt;
  a.tiles = (uint32_t)tiles;
  a.bps = (uint32_t)bps;
  a.ysplit = ranges > 1 ? (uint32_t)(m * ns[0]) : 0u;
  hipError_t e = hipErrorInvalidValue;
  switch (fmt) {
    case W4_NF4_X_F16: e = launch_fx<kNF4, kF16>(a, wn, wm, kw, s); break;
    case W4_NF4_X_BF16: e = launch_fx<kNF4, kBF16>(a, wn, wm, kw, s); break;
    case W4_INT4_X_F16: e = launch_fx<kINT4, kF16>(a, wn, wm, kw, s); break;
    case W4_INT4_X_BF16: e = launch_fx<kINT4, kBF16>(a, wn, wm, kw, s); break;
    case W4_FP4_X_F16: e = launch_fx<kFP4, kF16>(a, wn, wm, kw, s); break;
    case W4_FP4_X_BF16: e = launch_fx<kFP4, kBF16>(a, wn, wm, kw, s); break;
    case W4_INT4A_X_F16: e = launch_fx<kINT4A, kF16>(a, wn, wm, kw, s); break;
    case W4_INT4A_X_BF16: e = launch_fx<kINT4A, kBF16>(a, wn, wm, kw, s); break;
  }
  if (e != hipSuccess || ranges == 1) return e;
  // the ranges' partial sums, added in range order into y
  return launch_splitk_reduce(ws, y[0], m * ns[0], ranges, s);
}

hipError_t launch_gemm(int fmt, const uint16_t* x, const uint8_t* packed, const void* scales,
                       int64_t n, int64_t k, int64_t m, float* y, hipStream_t s, int splits,
                       float* ws) {
  return launch_gemm_members(fmt, x, 1, &packed, &scales, &n, &y, k, m, s, splits, ws);
}

}  // namespace w4
