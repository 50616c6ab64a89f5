// Kernel instantiations for one family (kept in its own translation unit so
// the three families compile in parallel).
#include "sk_dispatch.hpp"

namespace sk {
int launch_m2(int mode, int coef, int dk, int dv, int act, int sketch, const Params& p, hipStream_t st) {
  return launch_family<FAM_M2>(mode, coef, dk, dv, act, sketch, p, st);
}
}  // namespace sk
