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
// where c <= j).  16 rows per 256-thread workgroup.
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
constexpr int kRowsPerWg = 256 / kTeam;

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
  uint32_t code[kSlots];
  int t, bc, qmin;
  float fqmin, fqmax;
  const float* ut;
  const float* ud;
};

// Column J of the block: quantize it in its owner lane (divide, add the zero point, clamp, round,
// dequantize; e = (w - q_hat) / U_JJ), broadcast e over the 16-lane team, and subtract e U[J, c]
// (product rounded, then the subtraction) from the lane's columns c > J.
template <int J>
__device__ __forceinline__ void column_step(ColState& st) {
  constexpr int o = J & 15, mj = J >> 4;
  if (J >= st.bc) return;  // uniform
  const float wj = st.w[mj];
  float v = st.s[mj] != 0.0f ? div_rn(wj, st.s[mj]) : 0.0f;
  v = v + st.z[mj];
  v = fminf(fmaxf(v, st.fqmin), st.fqmax);
  const float q = rintf(v);
  const float qhat = (q - st.z[mj]) * st.s[mj];
  const float e_own = div_rn(wj - qhat, st.ud[J]);
  if (st.t == o) {
    st.qh[mj] = qhat;
    st.ee[mj] = e_own;
    st.code[mj] = (uint32_t)((int)q - st.qmin);
  }
  // DPP row broadcast of lane o of each 16-lane row: the owner's error to its team
  const float e = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, e_own), 0x150 + o, 0xF, 0xF, false));
  const float4 u0 = *reinterpret_cast<const float4*>(&st.ut[((J << 4) + st.t) * kSlots]);
  const float4 u1 = *reinterpret_cast<const float4*>(&st.ut[((J << 4) + st.t) * kSlots + 4]);
  const float uu[kSlots] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
  for (int m = mj; m < kSlots; ++m) {
    const float p = e * uu[m];
    // in slot mj the columns c <= J (lanes t <= o) keep their value
    if (m > mj || st.t > o) st.w[m] = st.w[m] - p;
  }
}

template <int... J>
__device__ __forceinline__ void run_columns(std::integer_sequence<int, J...>, ColState& st) {
  (column_step<J>(st), ...);
}

__global__ void __launch_bounds__(256) gptq_block_kernel(GptqBlockArgs a) {
  // U block, transposed: ut[(j * 16 + t) * 8 + m] = U[i1 + j, i1 + t + 16 m] for t + 16 m > j,
  // else 0; ud[j] = U[i1 + j, i1 + j].
  __shared__ __align__(16) float ut[kBlockMax * kTeam * kSlots];
  __shared__ float ud[kBlockMax];
  const int tid = threadIdx.x;
  const int bc = a.bc;
  for (int e = tid; e < kBlockMax * kBlockMax; e += 256) {
    const int j = e >> 7, c = e & 127;
    float v = 0.0f;
    if (j < bc && c < bc && c >= j) v = a.u[(int64_t)j * a.ldu + c];
    if (c == j) {
      ud[j] = v;
      v = 0.0f;
    }
    ut[((j << 4) + (c & 15)) * kSlots + (c >> 4)] = v;
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
    w[m] = in ? a.w[rr * a.ldw + c] : 0.0f;
    const int64_t g = (int64_t)((a.i1 + (in ? c : 0)) / a.group);
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
constexpr int kEPitch = kBlockMax + 1;

__global__ void __launch_bounds__(256) gptq_lazy_kernel(GptqLazyArgs a) {
  __shared__ float es[kTile * kEPitch];       // es[row * kEPitch + kk] = E[r0 + row, kk]
  __shared__ __align__(16) float us[kBlockMax * kTile];  // us[kk * 64 + col] = U[kk, c0 + col]
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kTile, c0 = (int64_t)blockIdx.y * kTile;
  const int bc = a.bc;
  for (int e = tid; e < kTile * kBlockMax; e += 256) {
    const int row = e >> 7, kk = e & 127;
    const int64_t r = r0 + row;
    es[row * kEPitch + kk] = (kk < bc && r < a.rows) ? a.err[r * a.lde + kk] : 0.0f;
  }
  for (int e = tid; e < kBlockMax * kTile; e += 256) {
    const int kk = e >> 6, col = e & 63;
    const int64_t c = c0 + col;
    us[kk * kTile + col] = (kk < bc && c < a.cols) ? a.u[(int64_t)kk * a.ldu + c] : 0.0f;
  }
  __syncthreads();
  const int tr = (tid >> 4) * 4, tc = (tid & 15) * 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[i][jj] = 0.0f;
  }
  for (int kk = 0; kk < bc; ++kk) {
    const float4 uv = *reinterpret_cast<const float4*>(&us[kk * kTile + tc]);
    const float ub[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ev = es[(tr + i) * kEPitch + kk];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float p = ev * ub[jj];
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
  hipLaunchKernelGGL(gptq_block_kernel, dim3((unsigned)grid), dim3(256), 0, s, a);
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
