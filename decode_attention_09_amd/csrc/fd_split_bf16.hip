// Split-kernel instantiations for bf16 inputs (head dims 16/32/64/128,
// 1..8 packed query rows). One file per element type so they compile in
// parallel.
#include "fd_split.h"

namespace fd {

hipError_t launch_split_bf16(const SplitArgs& a, int dim, int rows, bool mfma, dim3 grid,
                             hipStream_t s) {
  return launch_split_dt<DT_BF16>(a, dim, rows, mfma, grid, s);
}

}  // namespace fd
