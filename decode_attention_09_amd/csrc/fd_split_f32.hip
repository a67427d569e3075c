// Split-kernel instantiations for f32 inputs (head dims 16/32/64/128,
// 1..8 packed query rows). One file per element type so they compile in
// parallel.
#include "fd_split.h"

namespace fd {

hipError_t launch_split_f32(const SplitArgs& a, int dim, int rows, bool mfma, dim3 grid,
                             hipStream_t s) {
  return launch_split_dt<DT_F32>(a, dim, rows, mfma, grid, s);
}

}  // namespace fd
