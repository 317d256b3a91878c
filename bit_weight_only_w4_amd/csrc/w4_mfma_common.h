// Matrix-core building blocks shared by the MFMA kernels: the byte -> decoded-pair table in LDS,
// one 16x16x32 MFMA step on 16-bit fragments, and the DPP row broadcast that hands each lane the
// block scales of its D rows.  The decode follows the fused kernel of LLM Quantization on RTX 4060
// ("Kernel Implementation": read the packed bytes, look the codes up, scale per block); the table
// turns one packed byte into both of its weights with one LDS read.
#pragma once
#include "w4_common.h"

namespace w4 {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTableBytes = 32768;   // 256 entries x 128 bytes

__device__ inline uint32_t f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ inline uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Lane q (q < 16) receives the fp32 bits of table entry q of the NF4 or FP4 format.
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

// The byte -> decoded pair table, as in the GEMV kernel but with 32 copies of each 4-byte entry
// (16 of each 8-byte NF4 x bf16 entry): 128 bytes per entry, lane L reading copy L % 32 (L % 16).
// Half the GEMV's LDS, which leaves room for larger activation tiles.  Filled by all THREADS
// threads of a workgroup; the caller synchronizes before the first lookup.
template <int FMT, int XT, int THREADS>
__device__ inline void fill_table(uint32_t* tab) {
  uint32_t v1, v2 = 0;
  if (FMT == kFP4) {
    const float c = __uint_as_float(codes_in_lanes<kFP4>());  // exact in both 16-bit types
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
  constexpr bool kSplit = (FMT == kNF4 && XT == kBF16);
  uint4* t4 = reinterpret_cast<uint4*>(tab);
  const int tid = threadIdx.x;
  // 16-byte slot i belongs to entry i >> 3: high nibble i >> 7 (uniform over a wave), low nibble
  // (i >> 3) & 15 (the same for every slot of a thread).
  const uint32_t lo1 = (uint32_t)__shfl((int)v1, (tid >> 3) & 15) << 16;
  const uint32_t lo2 = kSplit ? (uint32_t)__shfl((int)v2, (tid >> 3) & 15) << 16 : 0u;
#pragma unroll 4
  for (int j = 0; j < kTableBytes / 16 / THREADS; ++j) {
    const int i = tid + THREADS * j;
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

// Lane i of each row of 16 lanes, broadcast to the row.  Every lane of a row reads a lane of that
// row, so the bound_ctrl form gives the same values and lets the compiler skip initializing the
// destination (one move per broadcast fewer).
template <int I>
__device__ inline float row_bcast(uint32_t v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x150 + I, 0xF, 0xF, true));
}

// Stages in LDS filled by buffer loads with the LDS destination: each wave's copies are counted
// by that wave's vmcnt, and a barrier does not wait for them, so before the barrier after which
// other waves read the stage, every wave waits for its own copies.
//
// wait_own_stage_copies reads one slot of the stage that this thread's copies filled.  The
// compiler makes an LDS read wait for the latest copy into the LDS object that holds it (all
// copies, if it cannot tell objects apart), and copies complete in issue order, so after the read
// every copy this wave issued into that object has landed.  The stage must be an LDS object of its
// own: waits are then only as long as this stage needs (the loads issued after its copies stay in
// flight).
__device__ inline void wait_own_stage_copies(const uint4* own_slot) {
  const uint4 v = *own_slot;
  asm volatile("" ::"v"(v.x));
}

// s_waitcnt vmcnt(0), the other counters left alone: for a stage whose copies are this wave's
// latest loads, where nothing is gained by naming the stage.
__device__ inline void wait_all_vector_loads() {
  // gfx9 encoding: vmcnt in bits 3:0 and 15:14 (0), expcnt 6:4 (7 = no wait), lgkmcnt 11:8 (15).
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

}  // namespace
}  // namespace w4
