// PowerSGD rank-r step, gfx950 (placeholder until the kernels land).
#include "common.hpp"
#include "internal.hpp"

namespace gc {

size_t powersgd_workspace(int64_t, int64_t, int) { return 0; }

hipError_t launch_powersgd(const float*, float*, int64_t, int64_t, int, float*, float*, void*,
                           hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace gc
