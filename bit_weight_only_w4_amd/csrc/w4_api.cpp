// C ABI of the W4 library: host-side validation, path and launch-shape selection, dispatch.
// Every check runs before any launch; nothing here allocates device memory or synchronizes a
// stream except the quantizers (which read back the device-side non-finite flag).
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "w4_common.h"

namespace w4 {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
      cus = 256;
    }
    cached[dev] = cus;
  }
  return cached[dev];
}

namespace {

struct CodebookInit {
  float v[16];
  CodebookInit() {
    const uint32_t bits[16] = W4_NF4_CODE_BITS;
    memcpy(v, bits, sizeof(v));
  }
};
const CodebookInit g_codebook;

// The quantizers and the 2:4 compression report non-finite weights through one device-side word
// each (per device), which a call resets, lets its kernel set, and reads back after synchronizing
// its stream.  Calls on different streams would otherwise interleave those three steps and lose or
// misattribute a flag, so the whole sequence runs under this lock (the calls synchronize anyway).
std::mutex g_flag_mu;

// Library settings that steer the automatic choices of w4_gemv and w4_gemm_smallbatch: a path
// override (w4_set_path, or W4_FORCE_PATH read once when the library loads) and a workspace
// registered per device (w4_set_workspace).  Guarded by g_settings_mu.
constexpr int kMaxDevices = 64;
struct Settings {
  int path = W4_PATH_AUTO;  // W4_PATH_AUTO = no override
  bool env_bad = false;     // W4_FORCE_PATH named no path: steered calls fail with W4_ERR_PATH
  void* ws[kMaxDevices] = {};
  size_t ws_bytes[kMaxDevices] = {};
};
std::mutex g_settings_mu;
Settings g_settings;

int parse_path_name(const char* v) {
  static const char* const names[] = {"auto", "gemv", "splitk", "mfma", "twopass", "tiled",
                                      "tiled_f16"};
  for (int i = 0; i < 7; ++i)
    if (strcmp(v, names[i]) == 0) return i;
  if (v[0] >= '0' && v[0] <= '6' && v[1] == 0) return v[0] - '0';
  return -1;
}

struct EnvInit {
  EnvInit() {
    const char* v = getenv("W4_FORCE_PATH");
    if (!v || !*v) return;
    const int p = parse_path_name(v);
    if (p < 0) {
      g_settings.env_bad = true;
    } else {
      g_settings.path = p;
    }
  }
};
const EnvInit g_env_init;

// The override and this device's registered workspace, read under the lock.
struct Steer {
  int path;
  bool bad;
  void* ws;
  size_t ws_bytes;
};
Steer current_steer() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  std::lock_guard<std::mutex> lock(g_settings_mu);
  Steer st{g_settings.path, g_settings.env_bad, nullptr, 0};
  if (dev >= 0) {
    st.ws = g_settings.ws[dev];
    st.ws_bytes = g_settings.ws_bytes[dev];
  }
  return st;
}

bool valid_fmt(int fmt) {
  return fmt == W4_NF4_X_F16 || fmt == W4_NF4_X_BF16 || fmt == W4_INT4_X_F16 ||
         fmt == W4_INT4_X_BF16 || fmt == W4_FP4_X_F16 || fmt == W4_FP4_X_BF16 ||
         fmt == W4_INT4A_X_F16 || fmt == W4_INT4A_X_BF16;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;

// Common matmul validation; returns W4_OK or the first failing check.
int validate(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t n,
             int64_t k, int64_t b, const float* y) {
  if (!valid_fmt(fmt)) return W4_ERR_FORMAT;
  if (!x || !packed || !scales || !y) return W4_ERR_NULL;
  const int64_t g = fmt_group(fmt);
  if (n < 1 || k < g || k % g != 0 || b < 1 || b > W4_MAX_BATCH || n >= kMaxDim || k >= kMaxDim)
    return W4_ERR_SHAPE;
  if (n > ((int64_t)1 << 62) / k) return W4_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 4)) return W4_ERR_ALIGN;
  if (!aligned(scales, fmt_scale_bytes(fmt))) return W4_ERR_ALIGN;
  const size_t ybytes = (size_t)(b * n) * 4;
  const size_t sbytes = (size_t)(n * (k / g)) * fmt_scale_bytes(fmt);
  if (overlaps(y, ybytes, x, (size_t)(b * k) * 2) || overlaps(y, ybytes, packed, (size_t)(n * k / 2)) ||
      overlaps(y, ybytes, scales, sbytes))
    return W4_ERR_ALIAS;
  return W4_OK;
}

// Whether the `used` bytes a path writes into the workspace overlap x, the packed weights or the
// scales (those kernels write partials or decoded weights while other workgroups still read them).
bool workspace_overlaps_inputs(const void* ws, size_t used, const void* x, const uint8_t* packed,
                               const void* scales, int fmt, int64_t n, int64_t k, int64_t b) {
  const size_t sbytes = (size_t)(n * (k / fmt_group(fmt))) * fmt_scale_bytes(fmt);
  return overlaps(ws, used, x, (size_t)(b * k) * 2) || overlaps(ws, used, packed, (size_t)(n * k / 2)) ||
         overlaps(ws, used, scales, sbytes);
}

int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// Launch shape of the fused GEMV for (N, K, B) over `splits` K ranges.
//
// The rules follow measurements on MI355X (graph replays of one shape over rotated copies):
//  * small matrices are latency-bound: give each lane as few 16-byte chunks as possible (one,
//    when a row has at most 64 chunks, else up to three) so that the first row block finishes
//    soon after its data lands;
//  * large matrices (>= 64 MiB of packed bytes) are bandwidth-bound: use narrow teams (16 lanes,
//    several rows per wave) and at most 256 workgroups of 512 threads that each stream many row
//    blocks, which keeps the per-lane activation footprint and the number of table fills small;
//  * at most two workgroups fit in one CU (64 KiB decode table each), so grids beyond two per CU
//    only queue.
bool plan_gemv(int64_t n, int64_t k, int b, int splits, GemvPlan* out, bool grouped = false) {
  const int cpr = (int)(k / 32);
  if (splits < 1 || splits > cpr) return false;
  // The kernel addresses a row block, the activations and their scales with 32-bit byte offsets
  // inside range-checked buffer resources: keep 32 rows of packed bytes below 2^31.
  if (k >= ((int64_t)1 << 26)) return false;
  const int cps = (cpr + splits - 1) / splits;
  if ((int64_t)(splits - 1) * cps >= cpr) return false;  // every split must own a chunk
  const int itmax = gemv_max_iters(b, grouped);
  const bool large = (n * (k / 2)) / splits >= ((int64_t)64 << 20);
  int team;
  if (large) {
    team = std::max(16, next_pow2((cps + 2) / 3));
  } else if (cps <= 64) {
    team = std::max(16, next_pow2(cps));
  } else {
    team = std::max(64, next_pow2((cps + 2) / 3));
  }
  while (team < kGemvMaxThreads && (cps + team - 1) / team > itmax) team *= 2;
  const int iters = (cps + team - 1) / team;
  if (iters > itmax) return false;
  GemvPlan p{};
  p.team = team;
  p.iters = iters;
  p.threads = (team >= 128 && !large) ? 256 : kGemvMaxThreads;
  if (p.threads < team) p.threads = team;
  p.splits = splits;
  p.cps = cps;
  const int64_t rows_per_wg = p.threads / p.team;
  const int64_t nrb = (n + rows_per_wg - 1) / rows_per_wg;
  const int64_t cus = device_cu_count();
  const int64_t cap = std::max<int64_t>(1, (large ? cus : 2 * cus) / splits);
  p.cap = (int)cap;
  p.grid_x = (int)std::min<int64_t>(nrb, cap);
  *out = p;
  return true;
}

// Split count the automatic path uses.  Measured on the 1536 x 8960 down projection, one pass
// with 128-lane teams beats every split-K configuration (the extra reduce launch costs more than
// the parallelism it adds), so the automatic choice is a single pass; split-K stays available
// explicitly through W4_PATH_SPLITK.
int auto_splits(int64_t, int64_t, int) { return 1; }

size_t splitk_bytes(int64_t n, int64_t b, int s) { return (size_t)s * (size_t)b * (size_t)n * 4; }

int pow2_at_least(int64_t v) {
  int p = 1;
  while (p < v && p < (1 << 30)) p *= 2;
  return p;
}

// Split count of the automatic MFMA path (used when the caller's workspace holds the partial
// sums).  Rows of at most 12 quads (3072 weights) never split, nor batches above 64 (1536 x 8960
// at B = 128: 25.3 us split 16 ways against 24.5 unsplit), nor matrices with two 128-row tiles
// per CU (128256 x 8192 at B = 32: 205 us split 4 ways against 195 unsplit, the partial sums
// adding 12% to the traffic).  Longer rows split K into the
// smallest power of two of ranges that (a) keeps one range's activation window, held rows x K / S
// x 2 bytes, within 128 KiB, and (b) gives matrices of few rows two row tiles of 16 rows per CU;
// at most 16 ranges, each of at least two quads.  Measured on MI355X (NF4 x fp16, rotated
// weights, every S from 1 to 16): the rule's S is the best or within 6% of it on 1536 x 8960 at
// B = 4..32 (14.9 -> 11.8 us at B = 32), 8192 x 28672 at B = 4..32 (72.3 -> 45.2 us at B = 32),
// 8192 x 8192 at B = 4..32 and 1024 x 8192 at B = 8 and 32; 28672 x 8192 at B = 32 gets 56.4 us
// against 59.3 unsplit (49.1 at S = 8).  Non-power-of-two counts measured slower throughout.
int auto_mfma_splits(int64_t n, int64_t k, int64_t b) {
  const int64_t quads = (k + 255) / 256;
  if (quads <= 12 || b > 64 || (n + 127) / 128 >= 2 * device_cu_count()) return 1;
  const int64_t rows = std::min<int64_t>(b, 128);
  const int sx = pow2_at_least((rows * k * 2 + 131071) / 131072);
  const int sp = pow2_at_least((2 * device_cu_count() * 16 + n - 1) / n);
  int s = std::min(std::max(sx, sp), 16);
  while (s > 1 && quads / s < 2) s /= 2;
  return s;
}

// Split count of the automatic tiled GEMM (used when the caller's workspace holds the partial
// sums).  Where the folded-scale kernel's own rule applies (fp16 activations with NF4, INT4, FP4
// or asymmetric INT4 weights from 128 rows, gemm_fold_auto_splits), it gives S.  Otherwise the
// smallest power of two S for which ceil(N / 64) * ceil(B / 128) * S, the workgroups
// of 64-row tiles over all K ranges, reaches three quarters of the CUs, with at least 16 blocks
// of 64 weights per range and at most 16 ranges.  Measured on MI355X (NF4 x fp16, rotated weights,
// S = 1..16 at B = 128, 256, 512): the rule's S is the best or within 10% of it on 1536 x 8960
// (72.6 -> 45.5 us at B = 512, 73.3 -> 27.0 at 256, 74.4 -> 21.0 at 128), 1024 x 8192 (63.7 ->
// 25.9, 64.4 -> 18.9, 64.2 -> 18.7) and 8192 x 8192 at B = 128 (65.2 -> 45.4); rows of 1536
// weights and matrices with enough tiles stay whole (8960 x 1536 at B = 128: 17.6 us unsplit,
// 28.7 split in two; 151936 x 1536 slower with every split).  It gives up to 10% on 8192 x 28672
// at B = 512 (444 us against 400 at S = 2).
int auto_tiled_splits(int fmt, int64_t n, int64_t k, int64_t b) {
  const int fold = gemm_fold_auto_splits(fmt, n, k, b);  // fp16 activations: the folded kernel's
  if (fold > 0) return fold;
  const int64_t tiles = ((n + 63) / 64) * ((b + 127) / 128);
  const int64_t nb = k / 64;
  const int64_t want = (3 * (int64_t)device_cu_count() + 3) / 4;
  int s = 1;
  while (s < 16 && tiles * s < want && nb / (2 * s) >= 16) s *= 2;
  return s;
}

// Launch shape of one fused-GEMV launch over `groups` members that share K: the plan of their
// summed rows, each member's row blocks, and each member's workgroups along x (its share of the
// grid cap, at most its row blocks; grouped launches give the members consecutive ranges of x, so
// no workgroup is without work).
bool plan_members(int groups, const int64_t* n, int64_t k, int b, int splits, bool grouped,
                  GemvPlan* p, int64_t* nrb, int64_t* grid_g) {
  int64_t n_total = 0;
  for (int g = 0; g < groups; ++g) n_total += n[g];
  if (b > kMaxGemvBatch || !plan_gemv(n_total, k, b, splits, p, grouped)) return false;
  const int64_t rows_per_wg = p->threads / p->team;
  int64_t nrb_sum = 0;
  for (int g = 0; g < groups; ++g) {
    nrb[g] = (n[g] + rows_per_wg - 1) / rows_per_wg;
    nrb_sum += nrb[g];
  }
  if (groups == 1) {
    grid_g[0] = std::min<int64_t>(nrb[0], p->cap);
    p->grid_x = (int)grid_g[0];
    return true;
  }
  int64_t total = 0;
  for (int g = 0; g < groups; ++g) {
    const int64_t share = (p->cap * nrb[g] + nrb_sum / 2) / nrb_sum;
    grid_g[g] = std::max<int64_t>(1, std::min<int64_t>(nrb[g], share));
    total += grid_g[g];
  }
  p->grid_x = (int)total;
  return true;
}

// One fused-GEMV launch over `groups` members that share x and K (splits > 1 only for a single
// member), then the split-K reduction if any.
int run_gemv_members(const void* x, int groups, const uint8_t* const* packed,
                     const void* const* scales, const int64_t* n, float* const* y, int fmt,
                     int64_t k, int64_t b, int splits, void* ws, hipStream_t st) {
  GemvPlan p;
  int64_t nrb[kMaxGroup], grid_g[kMaxGroup];
  if (!plan_members(groups, n, k, (int)b, splits, groups > 1, &p, nrb, grid_g)) return W4_ERR_PATH;
  GemvArgs a;
  memset(&a, 0, sizeof(a));
  a.x = reinterpret_cast<const uint16_t*>(x);
  uint32_t wg0 = 0;
  for (int g = 0; g < kMaxGroup; ++g) a.m[g].wg0 = 0xFFFFFFFFu;  // unused slots match no workgroup
  for (int g = 0; g < groups; ++g) {
    a.m[g].packed = packed[g];
    a.m[g].scales = scales[g];
    a.m[g].out = splits == 1 ? y[g] : reinterpret_cast<float*>(ws);
    a.m[g].n = (uint32_t)n[g];
    a.m[g].nrb = (uint32_t)nrb[g];
    a.m[g].wg0 = wg0;
    a.m[g].grid = (uint32_t)grid_g[g];
    wg0 += (uint32_t)grid_g[g];
  }
  a.k = k;
  a.cpr = (int)(k / 32);
  a.cps = p.cps;
  a.team = p.team;
  a.iters = p.iters;
  // The small decode table (a quarter of the 64 KiB fill, lookups with up to 4-way bank
  // conflicts) for 4-byte entries always: measured on MI355X (NF4 x fp16 decode step, rotated
  // per-kind times) it is faster on every launch kind, q|k|v 3.27 -> 3.10 us, gate|up 6.86 ->
  // 6.59, down 5.50 -> 5.03, lm_head 24.6 -> 24.3, step 535 -> 509 us: the fill's stores and its
  // barrier sit on each workgroup's critical path, the lookups' conflicts mostly do not.  NF4 x
  // bf16's 8-byte entries (8 copies in the small table) only where each workgroup streams one row
  // block of one chunk per lane or runs 256 threads: there q|k|v 3.38 -> 3.18 us and down 5.89 ->
  // 5.57, while gate|up (7.56 -> 8.06) and lm_head (26.8 -> 35.3) lose to the conflicts.
  bool one_trip = p.iters == 1;
  for (int g = 0; g < groups; ++g) one_trip = one_trip && nrb[g] <= grid_g[g];
  a.small_table = fmt != W4_NF4_X_BF16 || one_trip || p.threads == 256 ? 1 : 0;
  if (launch_gemv(fmt, (int)b, a, groups, p, st) != hipSuccess) return W4_ERR_HIP;
  if (splits > 1) {
    if (launch_splitk_reduce(reinterpret_cast<const float*>(ws), y[0], b * n[0], splits, st) !=
        hipSuccess)
      return W4_ERR_HIP;
  }
  return W4_OK;
}

int run_gemv(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t n,
             int64_t k, int64_t b, float* y, int splits, void* ws, hipStream_t st) {
  return run_gemv_members(x, 1, &packed, &scales, &n, &y, fmt, k, b, splits, ws, st);
}

int run_twopass(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t n,
                int64_t k, int64_t b, float* y, void* ws, hipStream_t st) {
  uint16_t* w_hat = reinterpret_cast<uint16_t*>(ws);
  if (launch_dequant_f16(fmt, packed, scales, n, k, w_hat, st) != hipSuccess) return W4_ERR_HIP;
  if (launch_dense_gemv(fmt, reinterpret_cast<const uint16_t*>(x), w_hat, n, k, b, y, st) !=
      hipSuccess)
    return W4_ERR_HIP;
  return W4_OK;
}

int run_mfma(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t n,
             int64_t k, int64_t b, float* y, hipStream_t st, int splits = 1, void* ws = nullptr) {
  const hipError_t e = launch_mfma(fmt, reinterpret_cast<const uint16_t*>(x), packed, scales, n, k,
                                   b, y, st, splits, reinterpret_cast<float*>(ws));
  if (e == hipErrorNotSupported) return W4_ERR_PATH;
  return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

// The folded-scale GEMM on one matrix: unsplit, the automatic tile rows, or 128-row tiles where
// the automatic choice would take the block-scale kernel; over K ranges, 128-row tiles.
int run_tiled_f16(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t n,
                  int64_t k, int64_t b, float* y, hipStream_t st, int splits = 1, void* ws = nullptr) {
  if (!gemm_fold_format(fmt)) return W4_ERR_PATH;
  int rows = splits > 1 ? 0 : gemm_fold_tile_rows(fmt, &n, 1, k, b);
  if (rows == 0) rows = 128;
  const hipError_t e = launch_gemm_fold(fmt, reinterpret_cast<const uint16_t*>(x), 1, &packed,
                                        &scales, &n, &y, k, b, rows, st, splits,
                                        reinterpret_cast<float*>(ws));
  if (e == hipErrorNotSupported) return W4_ERR_PATH;
  return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

int run_tiled(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t n,
              int64_t k, int64_t b, float* y, hipStream_t st, int splits = 1, void* ws = nullptr) {
  const hipError_t e = launch_gemm(fmt, reinterpret_cast<const uint16_t*>(x), packed, scales, n, k,
                                   b, y, st, splits, reinterpret_cast<float*>(ws));
  if (e == hipErrorNotSupported) return W4_ERR_PATH;
  return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

// Batch size from which the automatic path prefers the MFMA kernel: 4; 3 for matrices of 64 MiB
// of packed bytes and more; 5 for matrices under 4 MiB.  Measured on MI355X (NF4 x fp16, INT4 x
// bf16): the MFMA kernel's time hardly moves between B = 1 and 16, the GEMV's grows with B (one
// dot2 per weight pair and activation row); on 8960 x 1536 the GEMV is still faster at B = 3 and
// slower from B = 4, on 151936 x 1536 slower from B = 3; on the small launches (256, 1536 and
// 2048 rows x 1536) it is still 0.1-0.3 us faster at B = 4 (q 4.29 against 4.43 us, INT4 k/v
// 3.91 against 4.25) and slower from B = 6.
constexpr int64_t kMfmaFromBatch = 4;
constexpr int64_t kMfmaFromBatchLarge = 3;
constexpr int64_t kMfmaFromBatchSmall = 5;

bool prefer_mfma(int64_t n, int64_t k, int64_t b) {
  const int64_t bytes = n * (k / 2);
  const bool large = bytes >= ((int64_t)64 << 20);
  const bool small = bytes < ((int64_t)4 << 20);
  return b >= (large ? kMfmaFromBatchLarge : small ? kMfmaFromBatchSmall : kMfmaFromBatch);
}

// The tiled GEMM from W4_TILED_FROM_BATCH activation rows, for matrices of W4_TILED_FROM_ROWS rows
// and more.  Measured on MI355X at 512 activation rows (NF4 x fp16, INT4 x bf16): tiled against
// MFMA 48 / 57 us on 8960 x 1536, 437 / 500 us on 151936 x 1536, 403 / 519 us on 28672 x 8192;
// with 1536 or 2048 rows the tiles of one pass do not fill the CUs and the MFMA path is faster
// (17 / 14 us on 1536 x 1536, 66 / 57 us on 1536 x 8960) unless K splits (below).
bool prefer_tiled(int64_t n, int64_t b) { return b >= W4_TILED_FROM_BATCH && n >= W4_TILED_FROM_ROWS; }

// Fewer rows from W4_TILED_FROM_BATCH: the tiled GEMM over K ranges when the rule above splits K
// and the workspace holds the partial sums (1536 x 8960 at 512 / 256 / 128 activation rows: 45.5 /
// 27.0 / 21.0 us against the MFMA path's 56.9 / 47.2 / 24.5; 1024 x 8192: 25.9 / 18.9 / 18.7
// against 51.3 / 23.2 / 22.3), else the MFMA path.
bool prefer_tiled_split(int fmt, int64_t n, int64_t k, int64_t b, size_t workspace_bytes,
                        int* splits) {
  if (b < W4_TILED_FROM_BATCH || b * n >= ((int64_t)1 << 32)) return false;
  const int s = auto_tiled_splits(fmt, n, k, b);
  const int ranges = s > 1 ? gemm_splits_used(k, s) : 1;
  if (ranges > 1 && workspace_bytes >= splitk_bytes(n, b, ranges)) {
    *splits = s;
    return true;
  }
  return false;
}

// Arguments of a grouped call: every member valid on its own, the members' summed rows in range,
// and no member's y overlapping another member's y, packed bytes or scales.
int validate_group(const void* x, int groups, const uint8_t* const* packed,
                   const void* const* scales, const int64_t* n, float* const* y, int fmt,
                   int64_t k, int64_t b) {
  if (!valid_fmt(fmt)) return W4_ERR_FORMAT;
  if (groups < 1 || groups > W4_MAX_GROUP) return W4_ERR_SHAPE;
  if (!packed || !scales || !n || !y) return W4_ERR_NULL;
  int64_t n_total = 0;
  for (int g = 0; g < groups; ++g) {
    const int st = validate(x, packed[g], scales[g], fmt, n[g], k, b, y[g]);
    if (st != W4_OK) return st;
    n_total += n[g];
  }
  if (n_total >= kMaxDim) return W4_ERR_SHAPE;
  const size_t sdiv = (size_t)fmt_group(fmt), ssz = fmt_scale_bytes(fmt);
  for (int g = 0; g < groups; ++g) {
    const size_t yb = (size_t)(b * n[g]) * 4;
    for (int h = 0; h < groups; ++h) {
      if (h == g) continue;
      if (overlaps(y[g], yb, y[h], (size_t)(b * n[h]) * 4) ||
          overlaps(y[g], yb, packed[h], (size_t)(n[h] * k / 2)) ||
          overlaps(y[g], yb, scales[h], (size_t)(n[h] * (k / (int64_t)sdiv)) * ssz))
        return W4_ERR_ALIAS;
    }
  }
  return W4_OK;
}

// A validated group: from B = W4_TILED_FROM_BATCH a tiled-GEMM launch per member of at least
// W4_TILED_FROM_ROWS rows and one MFMA launch over the others; below it one MFMA launch over all
// members (mfma), else one fused-GEMV launch, or an MFMA launch when the GEMV has no launch shape
// for (K, B).
int run_group(const void* x, int groups, const uint8_t* const* packed, const void* const* scales,
              const int64_t* n, float* const* y, int fmt, int64_t k, int64_t b, bool mfma,
              hipStream_t s) {
  if (mfma && b >= W4_TILED_FROM_BATCH) {
    const uint8_t* tp[kMaxGroup];
    const void* ts[kMaxGroup];
    int64_t tn[kMaxGroup];
    float* ty[kMaxGroup];
    const uint8_t* rp[kMaxGroup];
    const void* rs[kMaxGroup];
    int64_t rn[kMaxGroup];
    float* ry[kMaxGroup];
    int tiled = 0, rest = 0;
    for (int g = 0; g < groups; ++g) {
      if (prefer_tiled(n[g], b)) {
        tp[tiled] = packed[g];
        ts[tiled] = scales[g];
        tn[tiled] = n[g];
        ty[tiled] = y[g];
        ++tiled;
      } else {
        rp[rest] = packed[g];
        rs[rest] = scales[g];
        rn[rest] = n[g];
        ry[rest] = y[g];
        ++rest;
      }
    }
    if (tiled > 0) {
      // one tiled launch over those members' tiles (8960 x 1536 twice at 512 activation rows:
      // 74.8 us in one launch against 2 x 45.7 us)
      const hipError_t e = launch_gemm_members(fmt, reinterpret_cast<const uint16_t*>(x), tiled, tp,
                                               ts, tn, ty, k, b, s);
      if (e == hipErrorNotSupported) return W4_ERR_PATH;
      if (e != hipSuccess) return W4_ERR_HIP;
    }
    if (rest == 0) return W4_OK;
    const hipError_t e = launch_mfma_members(fmt, reinterpret_cast<const uint16_t*>(x), rest, rp, rs,
                                             rn, ry, k, b, s);
    if (e == hipErrorNotSupported) return W4_ERR_PATH;
    return e == hipSuccess ? W4_OK : W4_ERR_HIP;
  }
  GemvPlan p;
  int64_t nrb[kMaxGroup], grid_g[kMaxGroup];
  if (mfma || !plan_members(groups, n, k, (int)b, 1, groups > 1, &p, nrb, grid_g)) {
    const hipError_t e = launch_mfma_members(fmt, reinterpret_cast<const uint16_t*>(x), groups,
                                             packed, scales, n, y, k, b, s);
    if (e == hipErrorNotSupported) return W4_ERR_PATH;
    return e == hipSuccess ? W4_OK : W4_ERR_HIP;
  }
  return run_gemv_members(x, groups, packed, scales, n, y, fmt, k, b, 1, nullptr, s);
}

}  // namespace
}  // namespace w4

using namespace w4;

extern "C" {

int w4_version(void) { return 1; }

const float* w4_nf4_codebook(void) { return g_codebook.v; }

const char* w4_status_string(int status) {
  switch (status) {
    case W4_OK: return "ok";
    case W4_ERR_NULL: return "null pointer argument";
    case W4_ERR_SHAPE: return "invalid shape (N, K, B) for this format";
    case W4_ERR_ALIGN: return "misaligned pointer";
    case W4_ERR_FORMAT: return "unknown weight/activation format";
    case W4_ERR_NONFINITE: return "non-finite weight passed to quantize";
    case W4_ERR_WORKSPACE: return "workspace missing or too small";
    case W4_ERR_PATH: return "path not available for these arguments";
    case W4_ERR_HIP: return "HIP runtime error";
    case W4_ERR_ALIAS: return "output overlaps an input or the workspace";
  }
  return "unknown status";
}

int w4_quantize_nf4(const float* w, int64_t n, int64_t k, uint8_t* packed, float* absmax,
                    void* stream) {
  if (!w || !packed || !absmax) return W4_ERR_NULL;
  if (n < 1 || k < 64 || k % 64 != 0 || n >= kMaxDim || k >= kMaxDim) return W4_ERR_SHAPE;
  if (!aligned(w, 8) || !aligned(packed, 16) || !aligned(absmax, 4)) return W4_ERR_ALIGN;
  if (overlaps(w, (size_t)(n * k) * 4, packed, (size_t)(n * k / 2)) ||
      overlaps(w, (size_t)(n * k) * 4, absmax, (size_t)(n * k / 64) * 4) ||
      overlaps(packed, (size_t)(n * k / 2), absmax, (size_t)(n * k / 64) * 4))
    return W4_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_flag_mu);
  if (quantize_error_reset(s) != hipSuccess) return W4_ERR_HIP;
  if (launch_quantize_nf4(w, n, k, packed, absmax, s) != hipSuccess) return W4_ERR_HIP;
  int flag = 0;
  if (quantize_error_read(&flag, s) != hipSuccess) return W4_ERR_HIP;
  return flag ? W4_ERR_NONFINITE : W4_OK;
}

int w4_quantize_fp4(const float* w, int64_t n, int64_t k, uint8_t* packed, float* scale,
                    void* stream) {
  if (!w || !packed || !scale) return W4_ERR_NULL;
  if (n < 1 || k < 64 || k % 64 != 0 || n >= kMaxDim || k >= kMaxDim) return W4_ERR_SHAPE;
  if (!aligned(w, 8) || !aligned(packed, 16) || !aligned(scale, 4)) return W4_ERR_ALIGN;
  if (overlaps(w, (size_t)(n * k) * 4, packed, (size_t)(n * k / 2)) ||
      overlaps(w, (size_t)(n * k) * 4, scale, (size_t)(n * k / 64) * 4) ||
      overlaps(packed, (size_t)(n * k / 2), scale, (size_t)(n * k / 64) * 4))
    return W4_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_flag_mu);
  if (quantize_error_reset(s) != hipSuccess) return W4_ERR_HIP;
  if (launch_quantize_fp4(w, n, k, packed, scale, s) != hipSuccess) return W4_ERR_HIP;
  int flag = 0;
  if (quantize_error_read(&flag, s) != hipSuccess) return W4_ERR_HIP;
  return flag ? W4_ERR_NONFINITE : W4_OK;
}

int w4_quantize_int4_asym(const float* w, int64_t n, int64_t k, uint8_t* packed, uint32_t* words,
                          void* stream) {
  if (!w || !packed || !words) return W4_ERR_NULL;
  if (n < 1 || k < 128 || k % 128 != 0 || n >= kMaxDim || k >= kMaxDim) return W4_ERR_SHAPE;
  if (!aligned(w, 8) || !aligned(packed, 16) || !aligned(words, 4)) return W4_ERR_ALIGN;
  if (overlaps(w, (size_t)(n * k) * 4, packed, (size_t)(n * k / 2)) ||
      overlaps(w, (size_t)(n * k) * 4, words, (size_t)(n * k / 128) * 4) ||
      overlaps(packed, (size_t)(n * k / 2), words, (size_t)(n * k / 128) * 4))
    return W4_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_flag_mu);
  if (quantize_error_reset(s) != hipSuccess) return W4_ERR_HIP;
  if (launch_quantize_int4_asym(w, n, k, packed, words, s) != hipSuccess) return W4_ERR_HIP;
  int flag = 0;
  if (quantize_error_read(&flag, s) != hipSuccess) return W4_ERR_HIP;
  return flag ? W4_ERR_NONFINITE : W4_OK;
}

int w4_quantize_int4(const float* w, int64_t n, int64_t k, uint8_t* packed, uint16_t* scale,
                     void* stream) {
  if (!w || !packed || !scale) return W4_ERR_NULL;
  if (n < 1 || k < 128 || k % 128 != 0 || n >= kMaxDim || k >= kMaxDim) return W4_ERR_SHAPE;
  if (!aligned(w, 8) || !aligned(packed, 16) || !aligned(scale, 2)) return W4_ERR_ALIGN;
  if (overlaps(w, (size_t)(n * k) * 4, packed, (size_t)(n * k / 2)) ||
      overlaps(w, (size_t)(n * k) * 4, scale, (size_t)(n * k / 128) * 2) ||
      overlaps(packed, (size_t)(n * k / 2), scale, (size_t)(n * k / 128) * 2))
    return W4_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_flag_mu);
  if (quantize_error_reset(s) != hipSuccess) return W4_ERR_HIP;
  if (launch_quantize_int4(w, n, k, packed, scale, s) != hipSuccess) return W4_ERR_HIP;
  int flag = 0;
  if (quantize_error_read(&flag, s) != hipSuccess) return W4_ERR_HIP;
  return flag ? W4_ERR_NONFINITE : W4_OK;
}

size_t w4_workspace_bytes(int fmt, int64_t n, int64_t k, int64_t b, int path, int split_k) {
  if (!valid_fmt(fmt)) return 0;
  const int64_t g = fmt_group(fmt);
  if (n < 1 || k < g || k % g || b < 1 || b > W4_MAX_BATCH || n >= kMaxDim || k >= kMaxDim) return 0;
  switch (path) {
    case W4_PATH_SPLITK: return splitk_bytes(n, b, split_k > 1 ? split_k : 4);
    case W4_PATH_MFMA: return split_k > 1 ? splitk_bytes(n, b, split_k) : 0;
    case W4_PATH_TILED: {
      const int ranges = split_k > 1 && split_k <= W4_MAX_SPLIT_K ? gemm_splits_used(k, split_k) : 1;
      return ranges > 1 ? splitk_bytes(n, b, ranges) : 0;
    }
    case W4_PATH_TILED_F16: {
      if (!gemm_fold_format(fmt)) return 0;
      const int ranges =
          split_k > 1 && split_k <= W4_MAX_SPLIT_K ? gemm_fold_ranges(fmt, k, split_k, nullptr) : 1;
      return ranges > 1 ? splitk_bytes(n, b, ranges) : 0;
    }
    case W4_PATH_TWOPASS: return (size_t)n * (size_t)k * 2;
    case W4_PATH_AUTO: {
      int sk = 1;
      const int p = w4_auto_path(fmt, n, k, b, SIZE_MAX, &sk);
      if (p == W4_PATH_TILED) return sk > 1 ? splitk_bytes(n, b, gemm_splits_used(k, sk)) : 0;
      return (p == W4_PATH_SPLITK || p == W4_PATH_MFMA) && sk > 1 ? splitk_bytes(n, b, sk) : 0;
    }
    default: return 0;
  }
}

int w4_gemv_plan(int fmt, int64_t n, int64_t k, int64_t b, int split_k, int* threads, int* team,
                 int* iters, int* chunks_per_split, int* grid_x) {
  if (!valid_fmt(fmt)) return W4_ERR_FORMAT;
  const int64_t g = fmt_group(fmt);
  if (n < 1 || k < g || k % g || b < 1 || b > W4_MAX_BATCH || n >= kMaxDim || k >= kMaxDim)
    return W4_ERR_SHAPE;
  GemvPlan p;
  if (b > kMaxGemvBatch || split_k < 1 || !plan_gemv(n, k, (int)b, split_k, &p)) return W4_ERR_PATH;
  if (threads) *threads = p.threads;
  if (team) *team = p.team;
  if (iters) *iters = p.iters;
  if (chunks_per_split) *chunks_per_split = p.cps;
  if (grid_x) *grid_x = p.grid_x;
  return W4_OK;
}

int w4_gemv_grouped_plan(int fmt, int groups, const int64_t* n, int64_t k, int64_t b,
                         int* threads, int* team, int* iters, int* grid_x, int* grid_z) {
  if (!valid_fmt(fmt)) return W4_ERR_FORMAT;
  if (groups < 1 || groups > W4_MAX_GROUP) return W4_ERR_SHAPE;
  if (!n) return W4_ERR_NULL;
  const int64_t g = fmt_group(fmt);
  int64_t n_total = 0;
  for (int i = 0; i < groups; ++i) {
    if (n[i] < 1 || n[i] >= kMaxDim) return W4_ERR_SHAPE;
    n_total += n[i];
  }
  if (n_total >= kMaxDim || k < g || k % g || k >= kMaxDim || b < 1 || b > W4_MAX_BATCH)
    return W4_ERR_SHAPE;
  GemvPlan p;
  int64_t nrb[kMaxGroup], grid_g[kMaxGroup];
  if (!plan_members(groups, n, k, (int)b, 1, groups > 1, &p, nrb, grid_g)) return W4_ERR_PATH;
  if (threads) *threads = p.threads;
  if (team) *team = p.team;
  if (iters) *iters = p.iters;
  if (grid_x) *grid_x = p.grid_x;
  if (grid_z) *grid_z = 1;
  return W4_OK;
}

int w4_auto_path(int fmt, int64_t n, int64_t k, int64_t b, size_t workspace_bytes, int* split_k) {
  if (!valid_fmt(fmt)) return W4_ERR_FORMAT;
  const int64_t g = fmt_group(fmt);
  if (n < 1 || k < g || k % g || b < 1 || b > W4_MAX_BATCH || n >= kMaxDim || k >= kMaxDim)
    return W4_ERR_SHAPE;
  int s = 1;
  int path;
  GemvPlan p;
  if (prefer_tiled(n, b)) {
    path = W4_PATH_TILED;
    int st = 1;
    if (prefer_tiled_split(fmt, n, k, b, workspace_bytes, &st)) s = st;
  } else if (prefer_tiled_split(fmt, n, k, b, workspace_bytes, &s)) {
    path = W4_PATH_TILED;
  } else if (prefer_mfma(n, k, b) || !plan_gemv(n, k, (int)b, 1, &p)) {
    path = W4_PATH_MFMA;
    s = auto_mfma_splits(n, k, b);
    if (s > 1 && workspace_bytes < splitk_bytes(n, b, s)) s = 1;
  } else {
    s = auto_splits(n, k, (int)b);
    if (s > 1 && workspace_bytes >= splitk_bytes(n, b, s)) {
      path = W4_PATH_SPLITK;
    } else {
      s = 1;
      path = W4_PATH_GEMV;
    }
  }
  if (split_k) *split_k = s;
  return path;
}

int w4_matmul_ex(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t n,
                 int64_t k, int64_t b, float* y, int path, int split_k, void* workspace,
                 size_t workspace_bytes, void* stream) {
  int st = validate(x, packed, scales, fmt, n, k, b, y);
  if (st != W4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (workspace && !aligned(workspace, 16)) return W4_ERR_ALIGN;
  if (workspace && overlaps(y, (size_t)(b * n) * 4, workspace, workspace_bytes)) return W4_ERR_ALIAS;
  if (path == W4_PATH_AUTO) {
    int sk = 1;
    path = w4_auto_path(fmt, n, k, b, workspace ? workspace_bytes : 0, &sk);
    if (path < 0) return path;
    split_k = sk;
  }
  switch (path) {
    case W4_PATH_GEMV:
      return run_gemv(x, packed, scales, fmt, n, k, b, y, 1, nullptr, s);
    case W4_PATH_SPLITK: {
      if (b > kMaxGemvBatch) return W4_ERR_PATH;
      if (split_k == 0) split_k = 4;
      if (split_k < 2 || split_k > W4_MAX_SPLIT_K || split_k > k / 32) return W4_ERR_PATH;
      const size_t used = splitk_bytes(n, b, split_k);
      if (!workspace || workspace_bytes < used) return W4_ERR_WORKSPACE;
      if (workspace_overlaps_inputs(workspace, used, x, packed, scales, fmt, n, k, b))
        return W4_ERR_ALIAS;
      return run_gemv(x, packed, scales, fmt, n, k, b, y, split_k, workspace, s);
    }
    case W4_PATH_MFMA: {
      if (split_k <= 1) return run_mfma(x, packed, scales, fmt, n, k, b, y, s);
      if (split_k > W4_MAX_SPLIT_K) return W4_ERR_PATH;
      const size_t used = splitk_bytes(n, b, split_k);
      if (!workspace || workspace_bytes < used) return W4_ERR_WORKSPACE;
      if (workspace_overlaps_inputs(workspace, used, x, packed, scales, fmt, n, k, b))
        return W4_ERR_ALIAS;
      return run_mfma(x, packed, scales, fmt, n, k, b, y, s, split_k, workspace);
    }
    case W4_PATH_TILED: {
      if (split_k <= 1) return run_tiled(x, packed, scales, fmt, n, k, b, y, s);
      if (split_k > W4_MAX_SPLIT_K) return W4_ERR_PATH;
      const int ranges = gemm_splits_used(k, split_k);
      if (ranges <= 1) return run_tiled(x, packed, scales, fmt, n, k, b, y, s);
      const size_t used = splitk_bytes(n, b, ranges);
      if (!workspace || workspace_bytes < used) return W4_ERR_WORKSPACE;
      if (workspace_overlaps_inputs(workspace, used, x, packed, scales, fmt, n, k, b))
        return W4_ERR_ALIAS;
      return run_tiled(x, packed, scales, fmt, n, k, b, y, s, ranges, workspace);
    }
    case W4_PATH_TILED_F16: {
      if (!gemm_fold_format(fmt) || split_k > W4_MAX_SPLIT_K) return W4_ERR_PATH;
      const int ranges = split_k > 1 ? gemm_fold_ranges(fmt, k, split_k, nullptr) : 1;
      if (ranges <= 1) return run_tiled_f16(x, packed, scales, fmt, n, k, b, y, s);
      const size_t used = splitk_bytes(n, b, ranges);
      if (!workspace || workspace_bytes < used) return W4_ERR_WORKSPACE;
      if (workspace_overlaps_inputs(workspace, used, x, packed, scales, fmt, n, k, b))
        return W4_ERR_ALIAS;
      return run_tiled_f16(x, packed, scales, fmt, n, k, b, y, s, split_k, workspace);
    }
    case W4_PATH_TWOPASS: {
      const size_t used = (size_t)n * (size_t)k * 2;
      if (!workspace || workspace_bytes < used) return W4_ERR_WORKSPACE;
      if (workspace_overlaps_inputs(workspace, used, x, packed, scales, fmt, n, k, b))
        return W4_ERR_ALIAS;
      return run_twopass(x, packed, scales, fmt, n, k, b, y, workspace, s);
    }
  }
  return W4_ERR_PATH;
}

int w4_gemv(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t n, int64_t k,
            int64_t b, float* y, void* stream) {
  int st = validate(x, packed, scales, fmt, n, k, b, y);
  if (st != W4_OK) return st;
  if (b > kMaxGemvBatch) return W4_ERR_SHAPE;
  const Steer steer = current_steer();
  if (steer.bad) return W4_ERR_PATH;
  if (steer.path != W4_PATH_AUTO)
    return w4_matmul_ex(x, packed, scales, fmt, n, k, b, y, steer.path, 0, steer.ws, steer.ws_bytes,
                        stream);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  GemvPlan p;
  if (!plan_gemv(n, k, (int)b, 1, &p)) return run_mfma(x, packed, scales, fmt, n, k, b, y, s);
  return run_gemv(x, packed, scales, fmt, n, k, b, y, 1, nullptr, s);
}

int w4_matmul_splitk_noalloc(const void* x, const uint8_t* packed, const void* scales, int fmt,
                             int64_t n, int64_t k, int64_t b, float* y, int split_k, void* stream) {
  const int st = validate(x, packed, scales, fmt, n, k, b, y);
  if (st != W4_OK) return st;
  if (b > kMaxGemvBatch) return W4_ERR_PATH;
  if (split_k == 0) split_k = 4;
  if (split_k < 2 || split_k > W4_MAX_SPLIT_K || split_k > k / 32) return W4_ERR_PATH;
  if (splitk_bytes(n, b, split_k) > (size_t)W4_NOALLOC_SCRATCH_BYTES) return W4_ERR_WORKSPACE;
  void* ws = nullptr;
  if (splitk_scratch(&ws) != hipSuccess) return W4_ERR_HIP;
  return run_gemv(x, packed, scales, fmt, n, k, b, y, split_k, ws,
                  reinterpret_cast<hipStream_t>(stream));
}

int w4_gemv_grouped(const void* x, int groups, const uint8_t* const* packed,
                    const void* const* scales, const int64_t* n, float* const* y, int fmt,
                    int64_t k, int64_t b, void* stream) {
  int st = validate_group(x, groups, packed, scales, n, y, fmt, k, b);
  if (st != W4_OK) return st;
  if (b > kMaxGemvBatch) return W4_ERR_SHAPE;
  return run_group(x, groups, packed, scales, n, y, fmt, k, b, false,
                   reinterpret_cast<hipStream_t>(stream));
}

int w4_gemm_smallbatch_grouped(const void* x, int groups, const uint8_t* const* packed,
                               const void* const* scales, const int64_t* n, float* const* y,
                               int fmt, int64_t k, int64_t b, void* stream) {
  int st = validate_group(x, groups, packed, scales, n, y, fmt, k, b);
  if (st != W4_OK) return st;
  int64_t n_total = 0;
  for (int g = 0; g < groups; ++g) n_total += n[g];
  return run_group(x, groups, packed, scales, n, y, fmt, k, b,
                   b > kMaxGemvBatch || prefer_mfma(n_total, k, b),
                   reinterpret_cast<hipStream_t>(stream));
}

int w4_gemm_smallbatch(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t n,
                       int64_t k, int64_t b, float* y, void* stream) {
  const Steer steer = current_steer();
  if (steer.bad) return W4_ERR_PATH;
  return w4_matmul_ex(x, packed, scales, fmt, n, k, b, y, steer.path, 0, steer.ws, steer.ws_bytes,
                      stream);
}

int w4_set_path(int path) {
  if (path < W4_PATH_AUTO || path > W4_PATH_TILED_F16) return W4_ERR_PATH;
  std::lock_guard<std::mutex> lock(g_settings_mu);
  g_settings.path = path;
  g_settings.env_bad = false;
  return W4_OK;
}

int w4_get_path(void) {
  std::lock_guard<std::mutex> lock(g_settings_mu);
  return g_settings.env_bad ? W4_ERR_PATH : g_settings.path;
}

int w4_set_workspace(void* workspace, size_t bytes) {
  if (!workspace && bytes != 0) return W4_ERR_NULL;
  if (workspace && !aligned(workspace, 16)) return W4_ERR_ALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W4_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_settings_mu);
  g_settings.ws[dev] = workspace;
  g_settings.ws_bytes[dev] = workspace ? bytes : 0;
  return W4_OK;
}

int w4_gemm_prefill(const void* x, const uint8_t* packed, const void* scales, int fmt, int64_t n,
                    int64_t k, int64_t b, float* y, void* stream) {
  const int st = validate(x, packed, scales, fmt, n, k, b, y);
  if (st != W4_OK) return st;
  return run_tiled(x, packed, scales, fmt, n, k, b, y, reinterpret_cast<hipStream_t>(stream));
}

int w4_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return W4_ERR_NULL;
  if (bytes == 0 || bytes % 16) return W4_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(sink, 4)) return W4_ERR_ALIGN;
  return launch_probe_read(src, bytes, sink, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? W4_OK
             : W4_ERR_HIP;
}

int w4_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return W4_ERR_NULL;
  if (bytes == 0 || bytes % 16) return W4_ERR_SHAPE;
  if (!aligned(src, 16) || !aligned(dst, 16)) return W4_ERR_ALIGN;
  if (overlaps(src, bytes, dst, bytes)) return W4_ERR_ALIAS;
  return launch_probe_copy(src, dst, bytes, reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? W4_OK
             : W4_ERR_HIP;
}

namespace {

// Shared checks of the GPTQ calls; 0 when the arguments are usable.
int gptq_check(const float* w, const float* u, const float* scale, const float* zero, int64_t rows,
               int64_t cols, int64_t group, int qmin, int qmax, const float* q_hat,
               const uint8_t* codes, const float* err) {
  if (!w || !u || !scale || !zero || !q_hat || !codes || !err) return W4_ERR_NULL;
  if (rows < 1 || cols < 1 || rows >= kMaxDim || cols >= ((int64_t)1 << 22)) return W4_ERR_SHAPE;
  if (group < 1 || cols % group != 0 || cols / group >= kMaxDim) return W4_ERR_SHAPE;
  if (qmin >= qmax || qmax - qmin > 255 || qmin < -32767 || qmax > 32767) return W4_ERR_SHAPE;
  if (!aligned(w, 4) || !aligned(u, 4) || !aligned(scale, 4) || !aligned(zero, 4) ||
      !aligned(q_hat, 4) || !aligned(err, 4))
    return W4_ERR_ALIGN;
  const size_t wb = (size_t)rows * (size_t)cols * 4, cb = (size_t)rows * (size_t)cols;
  const size_t ub = (size_t)cols * (size_t)cols * 4, sb = (size_t)rows * (size_t)(cols / group) * 4;
  const void* outs[3] = {q_hat, codes, err};
  const size_t outb[3] = {wb, cb, wb};
  const void* ins[4] = {w, u, scale, zero};
  const size_t inb[4] = {wb, ub, sb, sb};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps(outs[i], outb[i], ins[j], inb[j])) return W4_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlaps(outs[i], outb[i], outs[j], outb[j])) return W4_ERR_ALIAS;
  }
  for (int j = 1; j < 4; ++j)
    if (overlaps(w, wb, ins[j], inb[j])) return W4_ERR_ALIAS;
  return W4_OK;
}

int gptq_block(float* w, const float* u, const float* scale, const float* zero, int64_t rows,
               int64_t cols, int64_t group, int qmin, int qmax, int64_t col0, int64_t bcols,
               float* q_hat, uint8_t* codes, float* err, hipStream_t s) {
  const int64_t ng = cols / group;
  const hipError_t e = launch_gptq_block(
      w + col0, cols, u + col0 * cols + col0, cols, scale, zero, ng, (int)group,
      (int)col0, qmin, qmax, rows, (int)bcols, q_hat + col0, cols, codes + col0, cols, err + col0,
      cols, s);
  return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

int gptq_lazy(float* w, const float* u, const float* err, int64_t rows, int64_t cols, int64_t col0,
              int64_t bcols, hipStream_t s) {
  const int64_t i2 = col0 + bcols;
  if (i2 >= cols) return W4_OK;
  const hipError_t e = launch_gptq_lazy(w + i2, cols, err + col0, cols, u + col0 * cols + i2, cols,
                                        rows, cols - i2, (int)bcols, s);
  return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

// The lazy update of block [col0, col0 + bcols) restricted to columns [c_begin, c_end).
int gptq_lazy_range(float* w, const float* u, const float* err, int64_t rows, int64_t cols,
                    int64_t col0, int64_t bcols, int64_t c_begin, int64_t c_end, hipStream_t s) {
  if (c_begin >= c_end) return W4_OK;
  const hipError_t e = launch_gptq_lazy(w + c_begin, cols, err + col0, cols, u + col0 * cols + c_begin,
                                        cols, rows, c_end - c_begin, (int)bcols, s);
  return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

// Helper stream and events of w4_gptq_quantize on one device, created on the first call made
// outside stream capture (default priority, non-blocking).
struct GptqHelper {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool ok = false;
};
std::mutex g_gptq_mu;
GptqHelper g_gptq_helper[64];

GptqHelper* gptq_helper(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  GptqHelper& h = g_gptq_helper[dev];
  if (h.ok) return &h;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  if (hipStreamCreateWithFlags(&side, hipStreamNonBlocking) != hipSuccess) return nullptr;
  if (hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&join, hipEventDisableTiming) != hipSuccess) {
    if (fork) (void)hipEventDestroy(fork);
    (void)hipStreamDestroy(side);
    return nullptr;
  }
  h.side = side;
  h.fork = fork;
  h.join = join;
  h.ok = true;
  return &h;
}

}  // namespace

int w4_gptq_block_update(float* w, const float* u, const float* scale, const float* zero,
                         int64_t rows, int64_t cols, int64_t group, int qmin, int qmax,
                         int64_t col0, int64_t bcols, float* q_hat, uint8_t* codes, float* err,
                         void* stream) {
  const int st = gptq_check(w, u, scale, zero, rows, cols, group, qmin, qmax, q_hat, codes, err);
  if (st != W4_OK) return st;
  if (col0 < 0 || bcols < 1 || bcols > 128 || col0 + bcols > cols) return W4_ERR_SHAPE;
  return gptq_block(w, u, scale, zero, rows, cols, group, qmin, qmax, col0, bcols, q_hat, codes,
                    err, reinterpret_cast<hipStream_t>(stream));
}

int w4_gptq_lazy_update(float* w, const float* u, const float* err, int64_t rows, int64_t cols,
                        int64_t col0, int64_t bcols, void* stream) {
  if (!w || !u || !err) return W4_ERR_NULL;
  if (rows < 1 || cols < 1 || rows >= kMaxDim || cols >= ((int64_t)1 << 22)) return W4_ERR_SHAPE;
  if (col0 < 0 || bcols < 1 || bcols > 128 || col0 + bcols > cols) return W4_ERR_SHAPE;
  if (!aligned(w, 4) || !aligned(u, 4) || !aligned(err, 4)) return W4_ERR_ALIGN;
  const size_t wb = (size_t)rows * (size_t)cols * 4, ub = (size_t)cols * (size_t)cols * 4;
  if (overlaps(w, wb, u, ub) || overlaps(w, wb, err, wb)) return W4_ERR_ALIAS;
  return gptq_lazy(w, u, err, rows, cols, col0, bcols, reinterpret_cast<hipStream_t>(stream));
}

int w4_gptq_quantize(float* w, const float* u, const float* scale, const float* zero, int64_t rows,
                     int64_t cols, int64_t group, int qmin, int qmax, int64_t block, float* q_hat,
                     uint8_t* codes, float* err, void* stream) {
  const int st = gptq_check(w, u, scale, zero, rows, cols, group, qmin, qmax, q_hat, codes, err);
  if (st != W4_OK) return st;
  if (block < 1 || block > 128) return W4_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_gptq_mu);
  // Small layers keep one stream: the extra launches and the stream hand-offs cost more than the
  // overlap gains there (measured: q 1536 x 1536 and k 256 x 1536 slower, gate 8960 x 1536 and
  // down 1536 x 8960 faster with the helper stream).
  GptqHelper* h = rows * cols >= ((int64_t)1 << 23) ? gptq_helper(s) : nullptr;
  if (!h) {
    // one stream: each block, then its whole lazy update
    for (int64_t c0 = 0; c0 < cols; c0 += block) {
      const int64_t bc = std::min(block, cols - c0);
      int r = gptq_block(w, u, scale, zero, rows, cols, group, qmin, qmax, c0, bc, q_hat, codes, err, s);
      if (r != W4_OK) return r;
      r = gptq_lazy(w, u, err, rows, cols, c0, bc, s);
      if (r != W4_OK) return r;
    }
    return W4_OK;
  }
  // Two streams.  After block b, `s` updates only the next block's columns and goes on with the
  // next block's kernel, while the helper stream updates the columns beyond: the latency-bound
  // block kernel runs beside the lazy update.  Each column still takes the blocks' updates in
  // block order (`s` waits for the helper's previous update before its next narrow update), and
  // each update's arithmetic is unchanged, so the results are the same bits as on one stream.
  bool pending = false;  // a helper update not yet waited for
  // on an error, `stream` still joins the helper's pending work (a capture stays well formed)
  auto fail = [&](int code) {
    if (pending) (void)hipStreamWaitEvent(s, h->join, 0);
    return code;
  };
  for (int64_t c0 = 0; c0 < cols; c0 += block) {
    const int64_t bc = std::min(block, cols - c0);
    const int64_t i2 = c0 + bc, i3 = std::min(i2 + block, cols);
    int r = gptq_block(w, u, scale, zero, rows, cols, group, qmin, qmax, c0, bc, q_hat, codes, err, s);
    if (r != W4_OK) return fail(r);
    if (i2 >= cols) break;
    if (pending && hipStreamWaitEvent(s, h->join, 0) != hipSuccess) return fail(W4_ERR_HIP);
    pending = false;
    if (i3 < cols) {
      if (hipEventRecord(h->fork, s) != hipSuccess || hipStreamWaitEvent(h->side, h->fork, 0) != hipSuccess)
        return fail(W4_ERR_HIP);
      r = gptq_lazy_range(w, u, err, rows, cols, c0, bc, i3, cols, h->side);
      // the helper has work from here on (even if this launch failed, the wait below is needed)
      if (hipEventRecord(h->join, h->side) != hipSuccess) return W4_ERR_HIP;
      pending = true;
      if (r != W4_OK) return fail(r);
    }
    r = gptq_lazy_range(w, u, err, rows, cols, c0, bc, i2, i3, s);
    if (r != W4_OK) return fail(r);
  }
  if (pending && hipStreamWaitEvent(s, h->join, 0) != hipSuccess) return W4_ERR_HIP;
  return W4_OK;
}

int w4_sparse24_compress(const float* w, int64_t n, int64_t k, int xtype, uint16_t* values,
                         uint8_t* meta, void* stream) {
  if (!w || !values || !meta) return W4_ERR_NULL;
  if (xtype != W4_S24_F16 && xtype != W4_S24_BF16) return W4_ERR_FORMAT;
  if (n < 1 || k < 32 || k % 32 != 0 || k > 16384 || n >= kMaxDim) return W4_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(values, 16) || !aligned(meta, 4)) return W4_ERR_ALIGN;
  const size_t wb = (size_t)(n * k) * 4, vb = (size_t)(n * k), mb = (size_t)(n * k / 8);
  if (overlaps(w, wb, values, vb) || overlaps(w, wb, meta, mb) || overlaps(values, vb, meta, mb))
    return W4_ERR_ALIAS;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_flag_mu);
  if (sparse24_error_reset(s) != hipSuccess) return W4_ERR_HIP;
  if (launch_sparse24_compress(xtype, w, n, k, values, meta, s) != hipSuccess) return W4_ERR_HIP;
  int flag = 0;
  if (sparse24_error_read(&flag, s) != hipSuccess) return W4_ERR_HIP;
  return flag ? W4_ERR_NONFINITE : W4_OK;
}

int w4_sparse24_gemv(const uint16_t* x, const uint16_t* values, const uint8_t* meta, int xtype,
                     int64_t n, int64_t k, int64_t b, float* y, void* stream) {
  if (!x || !values || !meta || !y) return W4_ERR_NULL;
  if (xtype != W4_S24_F16 && xtype != W4_S24_BF16) return W4_ERR_FORMAT;
  if (n < 1 || k < 32 || k % 32 != 0 || k > 16384 || n >= kMaxDim || b < 1 || b > 8)
    return W4_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(values, 16) || !aligned(meta, 4) || !aligned(y, 4))
    return W4_ERR_ALIGN;
  const size_t yb = (size_t)(b * n) * 4;
  if (overlaps(y, yb, x, (size_t)(b * k) * 2) || overlaps(y, yb, values, (size_t)(n * k)) ||
      overlaps(y, yb, meta, (size_t)(n * k / 8)))
    return W4_ERR_ALIAS;
  const uint8_t* vp = reinterpret_cast<const uint8_t*>(values);
  const hipError_t e = launch_sparse24_gemv(xtype, x, 1, &vp, &meta, &n, &y, k, b,
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

int w4_sparse24_gemv_grouped(const uint16_t* x, int groups, const uint16_t* const* values,
                             const uint8_t* const* meta, const int64_t* N, int xtype, int64_t k,
                             int64_t b, float* const* y, void* stream) {
  if (!x || !values || !meta || !N || !y) return W4_ERR_NULL;
  if (groups < 1 || groups > W4_MAX_GROUP) return W4_ERR_SHAPE;
  if (xtype != W4_S24_F16 && xtype != W4_S24_BF16) return W4_ERR_FORMAT;
  if (k < 32 || k % 32 != 0 || k > 16384 || b < 1 || b > 8) return W4_ERR_SHAPE;
  if (!aligned(x, 16)) return W4_ERR_ALIGN;
  int64_t total = 0;
  const uint8_t* vps[W4_MAX_GROUP];
  for (int g = 0; g < groups; ++g) {
    if (!values[g] || !meta[g] || !y[g]) return W4_ERR_NULL;
    if (N[g] < 1) return W4_ERR_SHAPE;
    total += N[g];
    if (!aligned(values[g], 16) || !aligned(meta[g], 4) || !aligned(y[g], 4)) return W4_ERR_ALIGN;
    vps[g] = reinterpret_cast<const uint8_t*>(values[g]);
  }
  if (total >= kMaxDim) return W4_ERR_SHAPE;
  for (int g = 0; g < groups; ++g) {
    const size_t yb = (size_t)(b * N[g]) * 4;
    if (overlaps(y[g], yb, x, (size_t)(b * k) * 2)) return W4_ERR_ALIAS;
    for (int h = 0; h < groups; ++h) {
      if (overlaps(y[g], yb, values[h], (size_t)(N[h] * k)) ||
          overlaps(y[g], yb, meta[h], (size_t)(N[h] * k / 8)))
        return W4_ERR_ALIAS;
      if (h != g && overlaps(y[g], yb, y[h], (size_t)(b * N[h]) * 4)) return W4_ERR_ALIAS;
    }
  }
  const hipError_t e = launch_sparse24_gemv(xtype, x, groups, vps, meta, N, y, k, b,
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

}  // extern "C"
