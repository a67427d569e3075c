// Stand-ins for the kernel launchers of libfd, for the host-only sanitizer
// build of the C ABI (tests/test_host_sanitizers.py): that build instruments
// the host layer alone, and its checks never reach a launch. Any call here
// reports an error, so a check that did launch would fail its test.
#include "fd_internal.h"

namespace fd {

hipError_t launch_split_f32(const SplitArgs&, int, int, bool, dim3, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_split_f16(const SplitArgs&, int, int, bool, dim3, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_split_bf16(const SplitArgs&, int, int, bool, dim3, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_combine(const CombineArgs&, int, int, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_queue_reset(int*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_steal_reset(unsigned long long*, int, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace fd
