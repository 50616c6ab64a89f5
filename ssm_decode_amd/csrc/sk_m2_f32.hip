// Kernel instantiations of one family for fp32 activations and sketch.
#include "sk_dispatch.hpp"

namespace sk {
int launch_m2_f32(int mode, int coef, int dk, int dv, const Params& p, hipStream_t st) {
  return launch_dtype<FAM_M2, float, float>(mode, coef, dk, dv, p, st);
}
}  // namespace sk
