// MFMA path: host side (launch planning) and the single-matrix instantiations; the kernel is in
// w4_mfma_impl.h, the grouped instantiations in w4_mfma_grouped.hip.
#include "w4_mfma_impl.h"

namespace w4 {

// Launch shape of the MFMA kernel for one batch slice of T tiles.  K groups split K inside a
// workgroup when N alone gives too few row tiles: the smallest KW of 1, 2, 4, 8 that gives a row
// tile per CU (counting the batch slices).  The x window holds the slice's rows and as many quads
// per K group as fit the LDS next to the table and the reduction area, in phases of equal size.
// Every workgroup of the launch is resident at once: the grid is at most what fits the GPU (from
// the runtime's occupancy for the LDS in use), and a workgroup walks several row tiles when there
// are more tiles than that.
struct MfmaPlan {
  int tiles, kw, qpk, qpp, xrow, red, lds, ntiles, slices, qps, splits;
};

// Row tiles of `rows` rows over the members of a launch.
int64_t member_tiles(const int64_t* ns, int groups, int64_t rows) {
  int64_t t = 0;
  for (int g = 0; g < groups; ++g) t += (ns[g] + rows - 1) / rows;
  return t;
}

bool plan_slice(const int64_t* ns, int groups, int64_t k, int64_t b, int t, int splits,
                MfmaPlan* p) {
  // With split-K the rules below see one split's quads and count every split's workgroups.
  const int64_t quads_all = (k + kQuad - 1) / kQuad;
  splits = (int)std::max<int64_t>(1, std::min<int64_t>(splits, quads_all));
  const int64_t quads = (quads_all + splits - 1) / splits;
  const int64_t cus = device_cu_count();
  const int slices = (int)((b + 16 * t - 1) / (16 * t)) * splits;
  const int64_t rows_held = std::min<int64_t>(16 * t, b);
  int kw = 1;
  if (quads <= 12 && splits == 1) {
    // Rows of at most 3072 weights (measured on MI355X over the 1536-wide decode shapes at
    // B = 4..32): with one batch tile, eight K groups (one quad per wave, idle groups past K
    // reading zeros) beat fewer on every matrix that does not keep each resident workgroup busy
    // for two row tiles at one K group, where one K group is best (lm_head); with two or more
    // batch tiles (one workgroup per CU), the most K groups whose tiles still fit one round of
    // resident workgroups (a second, partial round costs more than the shorter waves save).
    if (t == 1) {
      kw = member_tiles(ns, groups, 16 * 8) * slices >= 2 * 2 * cus ? 1 : 8;
    } else {
      for (int c = max_kw(t); c >= 1; c /= 2) {
        kw = c;
        if (member_tiles(ns, groups, 16 * (8 / c)) * slices <= cus) break;
      }
    }
  } else {
    // Longer rows, or split-K (whose splits already supply the parallelism): the fewest K groups
    // that give every CU a row tile, which keeps row tiles tall and each activation loaded into
    // the window serving the most weight rows.
    for (int c = 1; c <= max_kw(t); c *= 2) {
      if (c > quads) break;
      kw = c;
      if (member_tiles(ns, groups, 16 * (8 / c)) * slices >= cus) break;
    }
  }
  const int64_t qpk = (quads + kw - 1) / kw;
  const int64_t red = kw > 1 ? (int64_t)(kw - 1) * (8 / kw) * t * 1024 : 0;
  const int64_t budget = kLdsBytes - kTableBytes - red;  // the table is static LDS
  int64_t qpp = qpk;
  // Window bytes, rounded up to whole rounds of 512 16-byte slots (each thread's last load may land
  // past the slots in use, inside the allocation).
  auto window = [&](int64_t q) {
    const int64_t slots = rows_held * ((int64_t)kw * 32 * q + 1);
    return (slots + kThreads - 1) / kThreads * kThreads * 16;
  };
  while (qpp > 1 && window(qpp) > budget) --qpp;
  if (window(qpp) > budget) return false;
  const int64_t nphase = (qpk + qpp - 1) / qpp;
  qpp = (qpk + nphase - 1) / nphase;  // the same number of phases, balanced
  p->tiles = t;
  p->kw = kw;
  p->qpk = (int)qpk;
  p->qpp = (int)qpp;
  p->xrow = (int)(((int64_t)kw * 32 * qpp + 1) * 16);
  p->red = (int)red;
  p->lds = (int)(red + window(qpp));  // dynamic LDS
  p->ntiles = (int)member_tiles(ns, groups, 16 * (8 / kw));
  p->slices = slices / splits;
  // Split z owns quads [z qps, (z + 1) qps); the last one may run past K (reads zeros), none is
  // empty.
  p->qps = splits > 1 ? (int)(kw * qpk) : 0;
  p->splits = splits > 1 ? (int)((quads_all + p->qps - 1) / p->qps) : 1;
  return true;
}

// Batch tiles per slice: the largest T (8, 4, 2, 1; at most what B needs) whose launch has at
// least half a row tile per CU; slices beyond the first re-read the weights (mostly from L2).
// Offsets are 32-bit: a slice's activations (16 T K 2 bytes) and K itself are bounded below.
bool plan_mfma(const int64_t* ns, int groups, int64_t k, int64_t b, int splits, MfmaPlan* out) {
  int64_t n_total = 0;
  for (int g = 0; g < groups; ++g) n_total += ns[g];
  if (b < 1 || b > W4_MAX_BATCH || k >= ((int64_t)1 << 22) || n_total >= ((int64_t)1 << 31) ||
      16 * kMaxTiles * k * 2 >= ((int64_t)1 << 31))
    return false;
  const int64_t cus = device_cu_count();
  const int need = (int)std::min<int64_t>((b + 15) / 16, kMaxTiles);
  const int tmax = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
  bool found = false;
  MfmaPlan best{};
  for (int t = tmax; t >= 1; t /= 2) {
    MfmaPlan p;
    if (!plan_slice(ns, groups, k, b, t, splits, &p)) continue;
    if (!found || (int64_t)p.ntiles * p.slices > (int64_t)best.ntiles * best.slices) {
      best = p;
      found = true;
    }
    if ((int64_t)p.ntiles * p.slices * p.splits * 2 >= cus) {
      best = p;
      break;
    }
  }
  if (found) *out = best;
  return found;
}

// One launch over all B rows of x and all members: grid.y = batch slices of up to 16 T rows,
// row tiles of every member on grid.x.
hipError_t launch_mfma_members(int fmt, const uint16_t* x, int groups, const uint8_t* const* packed,
                               const void* const* scales, const int64_t* ns, float* const* y,
                               int64_t k, int64_t b, hipStream_t s, int splits, float* ws) {
  if (groups < 1 || groups > kMaxGroup) return hipErrorInvalidValue;
  if (splits > 1 && (groups != 1 || ws == nullptr)) return hipErrorInvalidValue;
  if (splits > 1 && b * ns[0] >= ((int64_t)1 << 32)) return hipErrorNotSupported;  // 32-bit planes
  MfmaPlan p;
  if (!plan_mfma(ns, groups, k, b, splits, &p)) return hipErrorNotSupported;
  MfmaArgs a;
  memset(&a, 0, sizeof(a));
  const int64_t rows = 16 * (8 / p.kw);
  uint32_t tile0 = 0;
  for (int g = 0; g < groups; ++g) {
    a.m[g].packed = packed[g];
    a.m[g].scales = scales[g];
    a.m[g].y = p.splits > 1 ? ws : y[g];
    a.m[g].n = (uint32_t)ns[g];
    a.m[g].tile0 = tile0;
    tile0 += (uint32_t)((ns[g] + rows - 1) / rows);
  }
  a.x = x;
  a.groups = (uint32_t)groups;
  a.k = (uint32_t)k;
  a.b = (uint32_t)b;
  a.qpk = (uint32_t)p.qpk;
  a.qpp = (uint32_t)p.qpp;
  a.xrow = (uint32_t)p.xrow;
  a.red_bytes = (uint32_t)p.red;
  a.tiles = (uint32_t)p.ntiles;
  a.qps = (uint32_t)p.qps;
  a.ysplit = p.splits > 1 ? (uint32_t)(b * ns[0]) : 0u;
  // One member runs the instantiations without member selection (fewer live scalar registers).
  auto run = [&](int op, int grid, int* out) {
    return groups > 1 ? mfma_dispatch_grouped(op, fmt, a, p.tiles, p.kw, p.lds, grid, p.slices, out, s)
                      : dispatch<false>(op, fmt, a, p.tiles, p.kw, p.lds, grid, p.slices, out, s);
  };
  int resident = 0;
  hipError_t e = run(0, 0, &resident);
  if (e != hipSuccess) return e;
  if (resident < 1) return hipErrorNotSupported;
  const int64_t fit =
      std::max<int64_t>(1, (int64_t)device_cu_count() * resident / (p.slices * p.splits));
  const int grid = (int)std::min<int64_t>(p.ntiles, fit);
  a.tiles_base = (uint32_t)(p.ntiles / grid);
  a.tiles_rem = (uint32_t)(p.ntiles % grid);
  e = run(1, grid, nullptr);
  if (e != hipSuccess || p.splits == 1) return e;
  // the splits' partial sums, added in split order (bitwise reproducible), overwrite y
  return launch_splitk_reduce(ws, y[0], b * ns[0], p.splits, s);
}

hipError_t launch_mfma(int fmt, const uint16_t* x, const uint8_t* packed, const void* scales,
                       int64_t n, int64_t k, int64_t b, float* y, hipStream_t s, int splits,
                       float* ws) {
  return launch_mfma_members(fmt, x, 1, &packed, &scales, &n, &y, k, b, s, splits, ws);
}

int mfma_splits_used(int64_t n, int64_t k, int64_t b, int splits) {
  if (splits <= 1) return 1;
  MfmaPlan p;
  if (!plan_mfma(&n, 1, k, b, splits, &p)) return 0;
  return p.splits;
}

}  // namespace w4
