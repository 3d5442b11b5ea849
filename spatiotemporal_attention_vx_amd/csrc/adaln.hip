// Per-token AdaLN modulation: instantiations and launch (the kernel and
// its statistics are described in adaln_kernel.h).
#include "adaln_kernel.h"

namespace vx {

hipError_t launch_adaln_per_token(const void* x, const void* shift, const void* scale, void* y,
                                  int64_t rows, int64_t hidden, float eps, bool xb, bool mb,
                                  bool yb, hipStream_t st) {
    return adaln_dispatch<false>(x, shift, scale, y, rows, rows, hidden, eps, xb, mb, yb, st);
}

}  // namespace vx
