// MFMA path: the instantiations that take several matrices sharing x in one launch (their row
// tiles numbered one after another; see MfmaMember).
#include "w4_mfma_impl.h"

namespace w4 {

hipError_t mfma_dispatch_grouped(int op, int fmt, const MfmaArgs& a, int tiles, int kw, int lds,
                                 int grid, int slices, int* out, hipStream_t s) {
  return dispatch<true>(op, fmt, a, tiles, kw, lds, grid, slices, out, s);
}

}  // namespace w4
