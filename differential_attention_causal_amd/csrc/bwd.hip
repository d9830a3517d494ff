// Backward pass (placeholder until the kernels land).
#include "common.h"
#include "launch.h"

namespace diffattn {

size_t bwd_workspace_floats(int64_t B, int64_t H, int64_t N, int d) {
  return static_cast<size_t>(B * H * N) * (2 + 2 * static_cast<size_t>(d)) + 4096;
}

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  (void)a;
  (void)s;
  return hipErrorNotSupported;
}

}  // namespace diffattn
