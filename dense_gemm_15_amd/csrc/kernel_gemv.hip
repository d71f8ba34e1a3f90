// kernel_gemv.hip -- few-row products (M small, e.g. one token's GEMV).
// Not instantiated yet: such shapes run on the tiled kernels.
#include "kernels.hpp"

namespace g15 {

int gemv_entries(const KernelEntry** out) {
  *out = nullptr;
  return 0;
}

}  // namespace g15
