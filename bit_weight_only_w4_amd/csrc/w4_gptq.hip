// GPTQ's column loop on the GPU: the fused lazy-block update and the update of the columns to its
// right (LLM Compressor 0.14: GPTQ's 15x speedup is one fused loop).
//
// Per lazy block of bc <= 128 columns [i1, i1 + bc) ("Three changes that make it fast", "The fused
// kernel"): every row walks the block's columns left to right; column j is divided by the scale,
// the zero point added, clamped to [qmin, qmax], rounded half to even, dequantized
// (q_hat = (q - z) s); its error e = (w_j - q_hat) / U_jj is stored, and e U_{j,c} is subtracted
// from the block's columns c > j.  Rows are independent once they share the column order, so they
// run in parallel; the columns of a row run in sequence.  Then the columns right of the block take
// the block's errors at once: W[:, i2:] -= E U[i1:i2, i2:].
//
// Arithmetic: every operation in fp32, rounded on its own, in the order above (each product
// rounded, then the subtraction; no fused multiply-add, like the page's kernel, which avoids them
// to match the eager loop bit for bit).  Divisions are correctly rounded.  The lazy update sums
// the block's products in column order before subtracting.  The results are then bitwise those of
// the same loop run elementwise in IEEE fp32.
//
// Block kernel layout: a team of 16 lanes (one DPP row) owns one weight row; lane t holds the
// block's columns t, t + 16, ..., t + 112 in registers.  Column j belongs to lane j % 16, which
// quantizes it; its error goes to the team by a DPP row broadcast, and every lane updates its own
// columns right of j with U[j, c] read from LDS (the block of U transposed to [j][t][m], zero
// where c <= j).  32 rows per 512-thread workgroup; two workgroups fit a CU's LDS.
//
// Lazy-update kernel: 64 x 64 output tiles, each of 256 threads computing 4 x 4 outputs from the
// block's errors and U's rows staged in LDS.
#include <utility>

#include "w4_common.h"

#pragma clang fp contract(off)

namespace w4 {
namespace {

constexpr int kBlockMax = 128;
constexpr int kTeam = 16;
constexpr int kSlots = kBlockMax / kTeam;  // columns per lane
constexpr int kBlockThreads = 512;
constexpr int kRowsPerWg = kBlockThreads / kTeam;

__device__ inline float div_rn(float a, float b) { return __fdiv_rn(a, b); }

struct GptqBlockArgs {
  float* w;            // block's first column of row 0; row pitch ldw
  const float* u;      // U[i1, i1]; row pitch ldu
  const float* scale;  // scale[r, g], row pitch lds; group g of block column j = (i1 + j) / group
  const float* zero;
  float* q_hat;        // pitch ldq, block's first column
  uint8_t* codes;      // pitch ldc
  float* err;          // pitch lde
  int64_t ldw, ldu, lds, ldq, ldc, lde;
  int64_t rows;
  int bc;              // block columns (1..128)
  int i1;              // first column of the block (for the group index)
  int group;
  int qmin, qmax;
};

// One row's state in the block kernel: this lane's 8 columns and their results.
struct ColState {
  float w[kSlots], s[kSlots], z[kSlots], qh[kSlots], ee[kSlots];
  float d[kSlots];  // U_cc of the lane's columns c (the divisor when the lane owns the column)
  float4 u0, u1;    // row J of the transposed U block for this lane, read one column ahead
  uint32_t code[kSlots];
  int t, bc, qmin;
  float fqmin, fqmax;
  const float* ut;
  const float* ud;
};

// Column J of the block: quantize it in its owner lane (q = rint(clamp(w / s + z)),
// q_hat = (q - z) s; e = (w - q_hat) / U_JJ), broadcast e over the 16-lane team, and subtract e U[J, c]
// (product rounded, then the subtraction) from the lane's columns c > J.
template <int J>
__device__ __forceinline__ void column_step(ColState& st) {
  constexpr int o = J & 15, mj = J >> 4;
  if (J >= st.bc) return;  // uniform
  // this column's U row (read during the previous column), and the next one's, read now so that
  // its LDS latency overlaps this column's divisions
  const float4 u0 = st.u0, u1 = st.u1;
  if constexpr (J + 1 < kBlockMax) {
    st.u0 = *reinterpret_cast<const float4*>(&st.ut[(((J + 1) << 4) + st.t) * kSlots]);
    st.u1 = *reinterpret_cast<const float4*>(&st.ut[(((J + 1) << 4) + st.t) * kSlots + 4]);
  }
  const float wj = st.w[mj];
  float v = st.s[mj] != 0.0f ? div_rn(wj, st.s[mj]) : 0.0f;
  v = v + st.z[mj];
  v = fminf(fmaxf(v, st.fqmin), st.fqmax);
  const float q = rintf(v);
  const float qhat = (q - st.z[mj]) * st.s[mj];
  const float e_own = div_rn(wj - qhat, st.d[mj]);
  const bool own = st.t == o;
  st.qh[mj] = own ? qhat : st.qh[mj];
  st.ee[mj] = own ? e_own : st.ee[mj];
  st.code[mj] = own ? (uint32_t)((int)q - st.qmin) : st.code[mj];
  // DPP row broadcast of lane o of each 16-lane row: the owner's error to its team
  const float e = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, e_own), 0x150 + o, 0xF, 0xF, false));
  const float uu[kSlots] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
  for (int m = mj; m < kSlots; ++m) {
    const float p = e * uu[m];
    const float wn = st.w[m] - p;
    // in slot mj the columns c <= J (lanes t <= o) keep their value
    st.w[m] = (m > mj || st.t > o) ? wn : st.w[m];
  }
}

template <int... J>
__device__ __forceinline__ void run_columns(std::integer_sequence<int, J...>, ColState& st) {
  (column_step<J>(st), ...);
}

__global__ void __launch_bounds__(kBlockThreads, 2) gptq_block_kernel(GptqBlockArgs a) {
  // U block, transposed: ut[(j * 16 + t) * 8 + m] = U[i1 + j, i1 + t + 16 m] for t + 16 m > j,
  // else 0; ud[j] = U[i1 + j, i1 + j].
  __shared__ __align__(16) float ut[kBlockMax * kTeam * kSlots];
  __shared__ float ud[kBlockMax];
  const int tid = threadIdx.x;
  const int bc = a.bc;
  // Thread tid fills column c = tid & 127 of rows j = (tid >> 7) + 4 i, i = 0..31: every load is
  // issued unconditionally (indices clamped into the block) before the first LDS write, so the 32
  // loads are in flight together; values outside the upper triangle are then replaced by 0.
  constexpr int kFill = kBlockMax * kBlockMax / kBlockThreads;
  constexpr int kJStep = kBlockThreads / kBlockMax;
  {
    const int c = tid & 127, j0 = tid >> 7;
    const int cl = c < bc ? c : bc - 1;
    float uv[kFill];
#pragma unroll
    for (int i = 0; i < kFill; ++i) {
      const int j = j0 + kJStep * i;
      const int jl = j < bc ? j : bc - 1;
      uv[i] = a.u[(int64_t)jl * a.ldu + cl];
    }
#pragma unroll
    for (int i = 0; i < kFill; ++i) {
      const int j = j0 + kJStep * i;
      const bool upper = j < bc && c < bc && c > j;
      if (c == j) ud[j] = j < bc ? uv[i] : 0.0f;
      ut[((j << 4) + (c & 15)) * kSlots + (c >> 4)] = upper ? uv[i] : 0.0f;
    }
  }

  const int t = tid & (kTeam - 1);
  const int64_t r = (int64_t)blockIdx.x * kRowsPerWg + (tid >> 4);
  const bool row_ok = r < a.rows;
  const int64_t rr = row_ok ? r : 0;  // rows past the end compute on row 0's data, store nothing
  float w[kSlots], s[kSlots], z[kSlots];
#pragma unroll
  for (int m = 0; m < kSlots; ++m) {
    const int c = t + kTeam * m;
    const bool in = c < bc;
    const int cl = in ? c : bc - 1;  // every load in bounds and unconditional
    const float wv = a.w[rr * a.ldw + cl];
    w[m] = in ? wv : 0.0f;
    const int64_t g = (int64_t)((a.i1 + cl) / a.group);
    s[m] = a.scale[rr * a.lds + g];
    z[m] = a.zero[rr * a.lds + g];
  }
  __syncthreads();

  ColState st;
  st.t = t;
  st.bc = bc;
  st.qmin = a.qmin;
  st.ut = ut;
  st.ud = ud;
#pragma unroll
  for (int m = 0; m < kSlots; ++m) {
    st.w[m] = w[m];
    st.s[m] = s[m];
    st.z[m] = z[m];
    st.qh[m] = 0.0f;
    st.ee[m] = 0.0f;
    st.code[m] = 0u;
  }
#pragma unroll
  for (int m = 0; m < kSlots; ++m) st.d[m] = ud[t + kTeam * m];
  st.u0 = *reinterpret_cast<const float4*>(&ut[t * kSlots]);
  st.u1 = *reinterpret_cast<const float4*>(&ut[t * kSlots + 4]);
  st.fqmin = (float)a.qmin;
  st.fqmax = (float)a.qmax;
  // one copy of the column step per column (slot and owner lane are constants in each), so that
  // every register index is static
  run_columns(std::make_integer_sequence<int, kBlockMax>{}, st);

  if (row_ok) {
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
      const int c = t + kTeam * m;
      if (c < bc) {
        a.w[r * a.ldw + c] = st.w[m];
        a.q_hat[r * a.ldq + c] = st.qh[m];
        a.codes[r * a.ldc + c] = (uint8_t)st.code[m];
        a.err[r * a.lde + c] = st.ee[m];
      }
    }
  }
}

struct GptqLazyArgs {
  float* w;            // W[:, i2]: the first column right of the block; pitch ldw
  const float* err;    // E[:, i1]; pitch lde
  const float* u;      // U[i1, i2]; pitch ldu
  int64_t ldw, lde, ldu;
  int64_t rows, cols;  // rows x columns right of the block
  int bc;
};

constexpr int kTile = 64;
constexpr int kEPitch = kTile + 4;  // es row pitch (floats): 16-byte rows, writes spread over banks

__global__ void __launch_bounds__(256) gptq_lazy_kernel(GptqLazyArgs a) {
  __shared__ __align__(16) float es[kBlockMax * kEPitch];  // es[kk * kEPitch + row] = E[r0 + row, kk]
  __shared__ __align__(16) float us[kBlockMax * kTile];  // us[kk * 64 + col] = U[kk, c0 + col]
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kTile, c0 = (int64_t)blockIdx.y * kTile;
  const int bc = a.bc;
  // Loads unconditional (indices clamped into range) and all issued before the LDS writes.
  {
    const int kk = tid & 127, row0 = tid >> 7;
    const int kkl = kk < bc ? kk : bc - 1;
    float ev[kTile / 2];
#pragma unroll
    for (int i = 0; i < kTile / 2; ++i) {
      const int64_t r = r0 + row0 + 2 * i;
      ev[i] = a.err[(r < a.rows ? r : a.rows - 1) * a.lde + kkl];
    }
#pragma unroll
    for (int i = 0; i < kTile / 2; ++i) {
      const int row = row0 + 2 * i;
      es[kk * kEPitch + row] = (kk < bc && r0 + row < a.rows) ? ev[i] : 0.0f;
    }
  }
  {
    const int col = tid & 63, kk0 = tid >> 6;
    const int64_t c = c0 + col;
    const int64_t cl = c < a.cols ? c : a.cols - 1;
    float uv[kBlockMax / 4];
#pragma unroll
    for (int i = 0; i < kBlockMax / 4; ++i) {
      const int kk = kk0 + 4 * i;
      uv[i] = a.u[(int64_t)(kk < bc ? kk : bc - 1) * a.ldu + cl];
    }
#pragma unroll
    for (int i = 0; i < kBlockMax / 4; ++i) {
      const int kk = kk0 + 4 * i;
      us[kk * kTile + col] = (kk < bc && c < a.cols) ? uv[i] : 0.0f;
    }
  }
  __syncthreads();
  const int tr = (tid >> 4) * 4, tc = (tid & 15) * 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = 0.0f;
  }
  // the block's columns in order kk = 0, 1, ...: each product rounded, then added
#pragma unroll 4
  for (int kk = 0; kk < bc; ++kk) {
    const float4 uv = *reinterpret_cast<const float4*>(&us[kk * kTile + tc]);
    const float4 evv = *reinterpret_cast<const float4*>(&es[kk * kEPitch + tr]);
    const float ub[4] = {uv.x, uv.y, uv.z, uv.w};
    const float eb[4] = {evv.x, evv.y, evv.z, evv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float p = eb[i] * ub[jj];
        acc[i][jj] = acc[i][jj] + p;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = r0 + tr + i;
    if (r >= a.rows) continue;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int64_t c = c0 + tc + jj;
      if (c < a.cols) {
        float* p = a.w + r * a.ldw + c;
        *p = *p - acc[i][jj];
      }
    }
  }
}

}  // namespace

hipError_t launch_gptq_block(float* w, int64_t ldw, const float* u, int64_t ldu, const float* scale,
                             const float* zero, int64_t lds, int group, int i1, int qmin, int qmax,
                             int64_t rows, int bc, float* q_hat, int64_t ldq, uint8_t* codes,
                             int64_t ldc, float* err, int64_t lde, hipStream_t s) {
  GptqBlockArgs a{w, u, scale, zero, q_hat, codes, err, ldw, ldu, lds, ldq, ldc, lde, rows, bc, i1,
                  group, qmin, qmax};
  const int64_t grid = (rows + kRowsPerWg - 1) / kRowsPerWg;
  hipLaunchKernelGGL(gptq_block_kernel, dim3((unsigned)grid), dim3(kBlockThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gptq_lazy(float* w, int64_t ldw, const float* err, int64_t lde, const float* u,
                            int64_t ldu, int64_t rows, int64_t cols, int bc, hipStream_t s) {
  GptqLazyArgs a{w, err, u, ldw, lde, ldu, rows, cols, bc};
  const dim3 grid((unsigned)((rows + kTile - 1) / kTile), (unsigned)((cols + kTile - 1) / kTile));
  hipLaunchKernelGGL(gptq_lazy_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace w4
