// Fused 4-bit dequantize-and-multiply GEMV for gfx950 (CDNA4), batch 1..8 (kernel templates; one
// translation unit per weight x activation format instantiates them).
//
// Operation (LLM Quantization on RTX 4060: Where 4-bit Decode Falls Behind FP16, "Kernel
// Implementation"): y[b, n] = sum_k x[b, k] * code(nibble[n, k]) * scale[n, block(k)], reading each
// packed byte once from HBM, decoding on chip and accumulating in fp32.
//
// Layout of the work:
//   * A "team" of T lanes (16..512) owns one output row.  Lane t of a team streams the 16-byte
//     chunks t, t + T, t + 2T, ... of the row (one global_load_dwordx4 each; consecutive lanes on
//     consecutive chunks).  A chunk is 32 weights: half an NF4/FP4 block or a quarter of an INT4
//     group, so each chunk needs exactly one scale.
//   * The lane keeps the activations of its chunks in VGPRs for the whole launch and walks the
//     row blocks of its workgroup (grid-stride) with the next two row blocks' packed bytes and
//     scales already in flight.  The loop is unrolled three times so that the three buffers rotate
//     by register renaming: no copy of a loaded register, hence no wait on an outstanding load,
//     until the data is consumed.
//   * Every load is unconditional and in bounds (out-of-range chunks and row blocks are clamped
//     to valid ones and skipped by index when computing), so no branch joins force early waits.
//   * Decode (NF4): a 256-entry table in LDS maps a packed byte to the pair (value of the high
//     nibble, value of the low nibble) in the activation's 16-bit type; one ds_read_b32 decodes two
//     weights.  Each entry owns 256 bytes of LDS.  The full table holds 64 copies of each entry,
//     copy c in bank c, lane L reading copy L, so the lookups of a wave never conflict; the small
//     one holds 16 copies (lane L reads copy L & 15; lanes 16 apart share a bank) and takes a
//     quarter of the stores to write, which the host prefers where the fill costs more than the
//     conflicts.  The LDS address, byte value * 256 + lane offset, is built by one v_perm_b32.
//     The table is written while the first loads are in flight.  FP4
//     needs no table: gfx950 converts a byte of two E2M1 codes to a 16-bit pair in one
//     instruction (the pair comes out odd k first, so FP4 holds its activation pairs swapped).
//   * Multiply: v_dot2_f32_f16 / v_dot2_f32_bf16 of the decoded pair with the activation pair
//     into fp32 (products of two 16-bit values are exact in fp32), then one fp32 FMA per chunk with
//     the block scale.  NF4 with bf16 activations splits each code into two bf16 terms (8-byte
//     entries, 32 copies): a single bf16 code is not accurate enough.
//   * Reduction over a team: DPP within 16 lanes, cross-row shuffles up to 64, and an LDS exchange
//     between the waves of a team wider than one wave.
#pragma once
#include "w4_common.h"

namespace w4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

constexpr int kTableBytes = 65536;  // 256 entries x 256 bytes

__device__ inline uint32_t f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ inline uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Lane q (q < 16) receives the fp32 bits of table entry q of the NF4 or FP4 format; the constants
// go lane by lane from scalar registers, so building the table needs no memory access.
template <int FMT>
__device__ inline uint32_t codes_in_lanes() {
  constexpr uint32_t kn[16] = W4_NF4_CODE_BITS;
  constexpr uint32_t kf[16] = W4_FP4_CODE_BITS;
  uint32_t v = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q)
    asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(FMT == kFP4 ? kf[q] : kn[q]), "i"(q));
  return v;
}

// The decoded 16-bit value(s) of nibble (lane & 15), meaningful in lanes 0..15: the fp16 code
// (NF4 x fp16), the bf16 hi/lo split of the code (NF4 x bf16), the FP4 code (exact in both 16-bit
// types), or q - 8 in the activation type (INT4, exact).
template <int FMT, int XT>
__device__ inline void lane_decode(uint32_t& v1, uint32_t& v2) {
  v2 = 0;
  if (FMT == kFP4) {
    const float c = __uint_as_float(codes_in_lanes<kFP4>());
    v1 = XT == kF16 ? f16_bits(c) : (__float_as_uint(c) >> 16);
  } else if (FMT == kNF4) {
    const float c = __uint_as_float(codes_in_lanes<kNF4>());
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
}

// Write the table.  Each entry has 256 bytes of LDS; the full table fills all of them (64 copies
// of a 4-byte entry, 32 of an 8-byte one: 16 slots of 16 bytes), the small one the first 64
// bytes (SPE = 4 slots: 16 or 8 copies), a quarter of the stores for launches whose workgroups
// look up too few bytes to notice the conflicts (lanes L, L + 16, L + 32, L + 48 then share a
// bank).  Thread t writes slots t, t + NT, ...; slot i belongs to entry i / SPE, whose high nibble
// (i / 16 SPE) is the same for the whole wave (read with v_readlane) and whose low nibble
// ((i / SPE) & 15) is fixed per lane when NT >= 256.
template <int FMT, int XT, int NT, int SPE>
__device__ inline void fill_table(uint32_t* tab) {
  constexpr int kShift = SPE == 16 ? 4 : 2;  // log2(SPE)
  uint32_t v1, v2;
  lane_decode<FMT, XT>(v1, v2);
  constexpr bool kSplit = (FMT == kNF4 && XT == kBF16);
  uint4* t4 = reinterpret_cast<uint4*>(tab);
  const int tid = threadIdx.x;
  uint32_t lo1 = 0, lo2 = 0;
  if (NT >= 256) {
    lo1 = (uint32_t)__shfl((int)v1, (tid >> kShift) & 15) << 16;
    if (kSplit) lo2 = (uint32_t)__shfl((int)v2, (tid >> kShift) & 15) << 16;
  }
#pragma unroll 4
  for (int j = 0; j < 256 * SPE / NT; ++j) {
    const int i = tid + NT * j;
    const int hi = __builtin_amdgcn_readfirstlane(i >> (kShift + 4));
    if (NT < 256) {
      lo1 = (uint32_t)__shfl((int)v1, (i >> kShift) & 15) << 16;
      if (kSplit) lo2 = (uint32_t)__shfl((int)v2, (i >> kShift) & 15) << 16;
    }
    const uint32_t p1 = (uint32_t)__builtin_amdgcn_readlane((int)v1, hi) | lo1;
    const int slot = SPE == 16 ? i : ((i >> 2) << 4) | (i & 3);
    if (kSplit) {
      const uint32_t p2 = (uint32_t)__builtin_amdgcn_readlane((int)v2, hi) | lo2;
      t4[slot] = make_uint4(p1, p2, p1, p2);
    } else {
      t4[slot] = make_uint4(p1, p1, p1, p1);
    }
  }
}

template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}

// Sum over a team of `team` (16..64) lanes inside one wave; every lane of the team gets the total.
// Within a row of 16 lanes by DPP; across rows by gfx950's lane swaps (v_permlane16_swap: rows 0
// and 1, 2 and 3; v_permlane32_swap: the two halves), VALU operations instead of LDS shuffles.
__device__ inline float team_sum_wave(float v, int team) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror: all 16 lanes of a row hold the row sum
  if (team >= 32) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(s[0]) + __uint_as_float(s[1]);  // row r: r + (r ^ 1)
  }
  if (team >= 64) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(s[0]) + __uint_as_float(s[1]);  // lane l: l + (l ^ 32)
  }
  return v;
}

// Bytes of one row's scales, and the byte offset of chunk `chunk`'s scale within the row.
// INT4A keeps its 32-bit word (bf16 scale | zero point << 16) in the float slot, decoded when used.
template <int FMT>
__device__ inline uint32_t scale_pitch(int64_t k) {
  return FMT == kINT4A ? (uint32_t)(k >> 7) * 4u
         : FMT == kINT4 ? (uint32_t)(k >> 7) * 2u
                        : (uint32_t)(k >> 6) * 4u;
}
template <int FMT>
__device__ inline uint32_t scale_offset(int chunk) {
  return FMT == kINT4A ? (uint32_t)(chunk >> 2) * 4u
         : FMT == kINT4 ? (uint32_t)(chunk >> 2) * 2u
                        : (uint32_t)(chunk >> 1) * 4u;
}
// The scale slot of a chunk as loaded: fp32 (NF4, FP4), the 32-bit word (INT4A, as float bits),
// or the 16 bf16 bits (INT4), widened to fp32 only where the scale is used (scale_value).  Widened
// at load time, the conversion of every prefetched row block's scales waited for their loads
// right away (0.2 us per small launch).
template <int FMT>
using ScaleSlot = typename std::conditional<FMT == kINT4, uint16_t, float>::type;
template <int FMT>
__device__ inline ScaleSlot<FMT> load_scale(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (FMT == kINT4) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  } else {
    return __uint_as_float(buffer_load32(r, off));
  }
}
template <int FMT>
__device__ inline float scale_value(ScaleSlot<FMT> slot) {
  if constexpr (FMT == kINT4) {
    return __uint_as_float((uint32_t)slot << 16);  // bf16 -> fp32, exact
  } else {
    return slot;
  }
}

// Launches decoded without the LDS table (no fill, no lookups): FP4, through gfx950's E2M1 ->
// 16-bit conversion (v_cvt_scalef32_pk_{f16,bf16}_fp4 with scale 1: exact, one instruction per
// packed byte).  INT4 and asymmetric INT4 keep the table everywhere: a table-free INT4 decode
// (nibbles placed in the mantissa of M + q, 1.75 VALU instructions per packed byte, the offset
// taken off per chunk through the activation sums) paid off only against the 64 KiB fill, and
// with the 16-copy table it measured slower in every step (INT4 x bf16 at B = 1 490.5 us with the
// table against 492.3, asymmetric INT4 503.5 against 508.1, INT4 at B = 2 610.6 against 622.7).
template <int FMT>
constexpr bool table_free() {
  return FMT == kFP4;
}

// The two FP4 weights of byte KB of packed dword w as one activation-type pair.  The conversion
// returns the low nibble's value (odd k) in the low half, so FP4 keeps its activation pairs swapped
// (odd k low) to match.
template <int XT, int KB>
__device__ inline uint32_t fp4_pair(uint32_t w) {
  if constexpr (XT == kF16) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, KB));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, KB));
  }
}

template <int FMT, int XT, int B, int ITM, int NT, bool GROUPED>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 2)))
gemv_kernel(GemvArgsT<GROUPED ? kMaxGroup : 1> a) {
  constexpr bool kTable = !table_free<FMT>();
  __shared__ __align__(16) uint32_t tab[kTable ? kTableBytes / 4 : 4];
  __shared__ float xwave[NT / 64][B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int team = a.team;
  const int tshift = __builtin_ctz((unsigned)team);
  const int tl = tid & (team - 1);
  const int team_id = tid >> tshift;
  const int teams_per_wg = NT >> tshift;
  const int c0 = blockIdx.y * a.cps;
  const int nck = min(a.cps, a.cpr - c0);
  const int64_t k = a.k;
  // This workgroup's member: grouped launches give each member its own range of workgroups
  // along x, found by selects over the member slots (every slot is fetched in the one batch of
  // scalar loads; indexing the slots by a loaded value would add a second, dependent batch).
  GemvMember mm = a.m[0];
  if constexpr (!GROUPED) {
    // (Taking these fields here makes the compiler fetch the whole argument block in one batch
    // with one wait; the decode-table switch otherwise came in a late second batch whose wait
    // delayed the table fill by a scalar-memory round trip.)
    asm volatile("" ::"s"(mm.packed), "s"(mm.n), "s"(mm.nrb), "s"(mm.grid), "s"(a.x),
                 "s"(a.small_table), "s"(a.team));
  }
  if constexpr (GROUPED) {
    // (The empty asm statements take every slot's fields first, so that the compiler fetches them
    // in one batch instead of loading the chosen slot after comparing.)
#pragma unroll
    for (int i = 0; i < (GROUPED ? kMaxGroup : 1); ++i) {
      asm volatile("" ::"s"(a.m[i].packed), "s"(a.m[i].scales), "s"(a.m[i].out), "s"(a.m[i].n),
                   "s"(a.m[i].nrb), "s"(a.m[i].wg0), "s"(a.m[i].grid), "s"(a.x), "s"(a.small_table));
    }
#pragma unroll
    for (int i = 1; i < (GROUPED ? kMaxGroup : 1); ++i) {
      const bool take = blockIdx.x >= a.m[i].wg0;
      mm.packed = take ? a.m[i].packed : mm.packed;
      mm.scales = take ? a.m[i].scales : mm.scales;
      mm.out = take ? a.m[i].out : mm.out;
      mm.n = take ? a.m[i].n : mm.n;
      mm.nrb = take ? a.m[i].nrb : mm.nrb;
      mm.wg0 = take ? a.m[i].wg0 : mm.wg0;
      mm.grid = take ? a.m[i].grid : mm.grid;
    }
  }
  // 32-bit index arithmetic for row blocks (the host guarantees N < 2^31); one 32-bit division
  // gives this workgroup's trip count.
  const uint32_t nrb = mm.nrb;
  const uint32_t grid = mm.grid;  // = gridDim.x for one member (read with the other arguments)
  const uint32_t rb0 = GROUPED ? blockIdx.x - mm.wg0 : blockIdx.x;
  // Row blocks of this workgroup (>= 1) and the last of them; computed after the first row
  // block's and the activations' loads are issued (those need neither), so that the division
  // does not delay them.
  uint32_t count = 1u, rb_last = rb0;

  // Chunk index of slot i for this lane within the split, and whether the lane has that chunk.
  auto chunk_at = [&](int i) { return tl + (i << tshift); };
  // Member descriptor of row block rbv and the block's first row.
  struct Where {
    const uint8_t* packed;
    const void* scales;
    float* out;
    uint32_t n;
    uint32_t row0;
  };
  auto where = [&](uint32_t rbv) {
    return Where{mm.packed, mm.scales, mm.out, mm.n, rbv * (uint32_t)teams_per_wg};
  };
  // Row block rbv's packed bytes and scales for this lane, through buffer resources that span
  // exactly the block's existing rows: rows past N and chunks past the split read as zero
  // without touching memory, and need no clamping or branch.
  const uint32_t pitch = (uint32_t)(k >> 1);  // packed bytes per row
  const uint32_t spitch = scale_pitch<FMT>(k);
  auto load_rb = [&](uint32_t rbv, uint4 (&p)[ITM], ScaleSlot<FMT> (&s)[ITM], bool clamp = true) {
    // A prefetch past this workgroup's last row block re-reads that block (an L2 hit) rather
    // than switching the resource off, which would need a per-block select of its size.  The
    // first row block needs no clamp (rb0 <= rb_last), so its loads do not wait for the trip
    // count's division.
    const Where w = where(!clamp || rbv < rb_last ? rbv : rb_last);
    uint32_t rows = w.n - w.row0;  // w.row0 < w.n: every row block up to rb_last exists
    rows = rows < (uint32_t)teams_per_wg ? rows : (uint32_t)teams_per_wg;
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(w.packed + (int64_t)w.row0 * pitch, rows * pitch);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(
        reinterpret_cast<const char*>(w.scales) + (int64_t)w.row0 * spitch, rows * spitch);
#pragma unroll
    for (int i = 0; i < ITM; ++i) {
      const int c = chunk_at(i);
      const bool have = c < nck;
      p[i] = buffer_load16_stream(
          rp, offset_or_oob(have, (uint32_t)team_id * pitch + (uint32_t)(c0 + c) * 16u));
      s[i] = load_scale<FMT>(
          rs, offset_or_oob(have, (uint32_t)team_id * spitch + scale_offset<FMT>(c0 + c)));
    }
  };

  // --- first row block, then this lane's activations, then the second row block
  uint4 pA[ITM], pB[ITM], pC[ITM];
  ScaleSlot<FMT> sA[ITM], sB[ITM], sC[ITM];
  load_rb(rb0, pA, sA, false);
  uint32_t xr[ITM][B][16];
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(B * k * 2));
#pragma unroll
  for (int i = 0; i < ITM; ++i) {
    const int c = chunk_at(i);
    const bool have = c < nck;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const uint32_t xo = offset_or_oob(have, (uint32_t)(b * k + (int64_t)(c0 + c) * 32) * 2u);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 v = buffer_load16(rx, xo + 16u * q);
        if constexpr (FMT == kFP4) {
          // the hardware FP4 conversion yields (odd k, even k) pairs: swap each activation pair
          v = make_uint4(__builtin_amdgcn_alignbit(v.x, v.x, 16), __builtin_amdgcn_alignbit(v.y, v.y, 16),
                         __builtin_amdgcn_alignbit(v.z, v.z, 16), __builtin_amdgcn_alignbit(v.w, v.w, 16));
        }
        xr[i][b][4 * q + 0] = v.x;
        xr[i][b][4 * q + 1] = v.y;
        xr[i][b][4 * q + 2] = v.z;
        xr[i][b][4 * q + 3] = v.w;
      }
    }
  }
  // (Table launches: the division after the loads above.  FP4 rearranges its activation pairs
  // as they arrive; a scheduling barrier here would make those rearrangements wait for the loads
  // before the next row block is requested, 1% slower per step.)
  if constexpr (kTable) __builtin_amdgcn_sched_barrier(0);
  count = (nrb - 1u - rb0) / grid + 1u;
  rb_last = rb0 + grid * (count - 1u);
  load_rb(rb0 + grid, pB, sB);


  // --- decode table, written while the loads above are in flight
  if constexpr (kTable) {
    if (a.small_table) {
      fill_table<FMT, XT, NT, 4>(tab);
    } else {
      fill_table<FMT, XT, NT, 16>(tab);
    }
    __syncthreads();
  }

  // INT4A: the sum of each chunk's 32 activations (per batch row), for the zero-point term
  // -(z - 8) * s * sum(x) of every row this lane meets; computed once per launch.
  constexpr bool kXsum = FMT == kINT4A;
  float xsum[kXsum ? ITM : 1][B];
  if constexpr (kXsum && kTable) {
    // Keep the sums behind the barrier: computed before it, they made every wave wait for its
    // activations (and the row block loaded ahead of them) before the barrier, which then waited
    // for the slowest wave's loads (0.3 us per small launch).
#pragma unroll
    for (int i = 0; i < ITM; ++i) {
#pragma unroll
      for (int b = 0; b < B; ++b) {
#pragma unroll
        for (int m = 0; m < 16; ++m) asm volatile("" : "+v"(xr[i][b][m]));
      }
    }
  }
  if constexpr (kXsum) {
    constexpr uint32_t kOnes = XT == kF16 ? 0x3C003C00u : 0x3F803F80u;
#pragma unroll
    for (int i = 0; i < ITM; ++i) {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float t = 0.0f;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          if (XT == kF16) {
            t = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, xr[i][b][m]),
                                       __builtin_bit_cast(half2_t, kOnes), t, false);
          } else {
            t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, xr[i][b][m]),
                                                __builtin_bit_cast(bf162_t, kOnes), t, false);
          }
        }
        xsum[i][b] = t;
      }
    }
  }

  constexpr bool kSplitCode = (FMT == kNF4 && XT == kBF16);
  // copy of this lane (see fill_table): 64 / 32 copies, or 16 / 8 in the small table
  const uint32_t cmask = a.small_table ? (kSplitCode ? 7u : 15u) : (kSplitCode ? 31u : 63u);
  const uint32_t laneoff = ((uint32_t)lane & cmask) * (kSplitCode ? 8u : 4u);
  const char* tabc = reinterpret_cast<const char*>(tab);
  const int wave = tid >> 6;
  const int waves_per_team = team > 64 ? team >> 6 : 1;

  auto compute_store = [&](uint32_t rbv, const uint4 (&pk)[ITM], const ScaleSlot<FMT> (&sc)[ITM]) {
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
            const int m = 4 * j + kb;  // byte index in the chunk = activation pair index
            if constexpr (!kTable) {
              const uint32_t t = kb == 0   ? fp4_pair<XT, 0>(wv[j])
                                 : kb == 1 ? fp4_pair<XT, 1>(wv[j])
                                 : kb == 2 ? fp4_pair<XT, 2>(wv[j])
                                           : fp4_pair<XT, 3>(wv[j]);
#pragma unroll
              for (int b = 0; b < B; ++b) {
                if (XT == kF16) {
                  d[b] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, t),
                                                __builtin_bit_cast(half2_t, xr[i][b][m]), d[b], false);
                } else {
                  d[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, t),
                                                         __builtin_bit_cast(bf162_t, xr[i][b][m]),
                                                         d[b], false);
                }
              }
              continue;
            }
            // LDS byte address: lane offset in byte 0, the packed byte in byte 1.
            const uint32_t addr =
                __builtin_amdgcn_perm(wv[j], laneoff, 0x0C0C0000u | ((4u + (uint32_t)kb) << 8));
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
                                                         __builtin_bit_cast(bf162_t, xr[i][b][m]),
                                                         d[b], false);
                }
              }
            }
          }
        }
        if constexpr (FMT == kINT4A) {
          // (q - z) s = ((q - 8) - (z - 8)) s: the table gives q - 8
          const uint32_t word = __float_as_uint(sc[i]);
          const float s = __uint_as_float(word << 16);
          const float zc = -8.0f + (float)((word >> 16) & 15u);
#pragma unroll
          for (int b = 0; b < B; ++b) acc[b] = __builtin_fmaf(__builtin_fmaf(-zc, xsum[i][b], d[b]), s, acc[b]);
        } else {
          const float s = scale_value<FMT>(sc[i]);
#pragma unroll
          for (int b = 0; b < B; ++b) acc[b] = __builtin_fmaf(d[b], s, acc[b]);
        }
      }
    }

    const Where w = where(rbv);
    const uint32_t row = w.row0 + (uint32_t)team_id;
    const int64_t n = w.n;
#pragma unroll
    for (int b = 0; b < B; ++b) acc[b] = team_sum_wave(acc[b], team);
    float* out = w.out + (int64_t)blockIdx.y * B * n;
    if (waves_per_team == 1) {
      if (tl == 0 && row < w.n) {
#pragma unroll
        for (int b = 0; b < B; ++b) out[b * n + row] = acc[b];
      }
    } else {
      if (lane == 0) {
#pragma unroll
        for (int b = 0; b < B; ++b) xwave[wave][b] = acc[b];
      }
      __syncthreads();
      if (tl == 0 && row < w.n) {
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float v = 0.0f;
          for (int w = 0; w < waves_per_team; ++w) v += xwave[wave + w][b];
          out[b * n + row] = v;
        }
      }
      __syncthreads();
    }
  };

  // --- main loop: three row blocks per trip, buffers rotating A -> B -> C, two row blocks in
  // flight behind the one being computed, no early exit; the last one or two row blocks are
  // already loaded when the loop ends.  (Requesting the third block before the table fill instead
  // measured slower on small matrices.)
  uint32_t rb = rb0;
  uint32_t t = 0;
  for (; t + 3 <= count; t += 3) {
    load_rb(rb + 2 * grid, pC, sC);
    compute_store(rb, pA, sA);
    load_rb(rb + 3 * grid, pA, sA);
    compute_store(rb + grid, pB, sB);
    load_rb(rb + 4 * grid, pB, sB);
    compute_store(rb + 2 * grid, pC, sC);
    rb += 3 * grid;
  }
  if (t < count) compute_store(rb, pA, sA);
  if (t + 1 < count) compute_store(rb + grid, pB, sB);
}

template <int FMT, int XT, int B, int ITM, bool GROUPED>
hipError_t launch_one(const GemvArgs& full, int groups, const GemvPlan& p, hipStream_t s) {
  constexpr int G = GROUPED ? kMaxGroup : 1;
  GemvArgsT<G> a;
  a.x = full.x;
  a.k = full.k;
  a.cpr = full.cpr;
  a.cps = full.cps;
  a.team = full.team;
  a.iters = full.iters;
  a.small_table = full.small_table;
  for (int g = 0; g < G; ++g) a.m[g] = full.m[g];
  (void)groups;
  const dim3 grid(p.grid_x, p.splits, 1);
  switch (p.threads) {
    case 256:
      hipLaunchKernelGGL((gemv_kernel<FMT, XT, B, ITM, 256, GROUPED>), grid, dim3(256), 0, s, a);
      break;
    case 512:
      hipLaunchKernelGGL((gemv_kernel<FMT, XT, B, ITM, 512, GROUPED>), grid, dim3(512), 0, s, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Chunks per lane instantiated for batch B: up to gemv_max_iters(B, GROUPED).
template <int FMT, int XT, int B, bool GROUPED>
hipError_t launch_b(const GemvArgs& a, int groups, const GemvPlan& p, hipStream_t s) {
  constexpr int kMax = gemv_max_iters(B, GROUPED);
  switch (p.iters) {
    case 1: return launch_one<FMT, XT, B, 1, GROUPED>(a, groups, p, s);
    case 2: if constexpr (kMax >= 2) return launch_one<FMT, XT, B, 2, GROUPED>(a, groups, p, s); break;
    case 3: if constexpr (kMax >= 3) return launch_one<FMT, XT, B, 3, GROUPED>(a, groups, p, s); break;
    case 4: if constexpr (kMax >= 4) return launch_one<FMT, XT, B, 4, GROUPED>(a, groups, p, s); break;
    case 5: if constexpr (kMax >= 5) return launch_one<FMT, XT, B, 5, GROUPED>(a, groups, p, s); break;
    case 6: if constexpr (kMax >= 6) return launch_one<FMT, XT, B, 6, GROUPED>(a, groups, p, s); break;
    case 7: if constexpr (kMax >= 7) return launch_one<FMT, XT, B, 7, GROUPED>(a, groups, p, s); break;
    case 8: if constexpr (kMax >= 8) return launch_one<FMT, XT, B, 8, GROUPED>(a, groups, p, s); break;
  }
  return hipErrorInvalidValue;
}

template <int FMT, int XT, bool GROUPED>
hipError_t launch_fx(int b, const GemvArgs& a, int groups, const GemvPlan& p, hipStream_t s) {
  switch (b) {
    case 1: return launch_b<FMT, XT, 1, GROUPED>(a, groups, p, s);
    case 2: return launch_b<FMT, XT, 2, GROUPED>(a, groups, p, s);
    case 3: return launch_b<FMT, XT, 3, GROUPED>(a, groups, p, s);
    case 4: return launch_b<FMT, XT, 4, GROUPED>(a, groups, p, s);
    case 5: return launch_b<FMT, XT, 5, GROUPED>(a, groups, p, s);
    case 6: return launch_b<FMT, XT, 6, GROUPED>(a, groups, p, s);
    case 7: return launch_b<FMT, XT, 7, GROUPED>(a, groups, p, s);
    case 8: return launch_b<FMT, XT, 8, GROUPED>(a, groups, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace w4
