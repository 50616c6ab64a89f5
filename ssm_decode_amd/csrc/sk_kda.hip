// Kernel instantiations of one family for bf16 activations and sketch, and
// the family's entry point (each family and dtype is its own translation
// unit, so that they compile in parallel).
#include "sk_dispatch.hpp"

namespace sk {
int launch_kda_f32(int mode, int coef, int dk, int dv, const Params& p, hipStream_t st);

int launch_kda(int mode, int coef, int dk, int dv, int act, int sketch, const Params& p, hipStream_t st) {
  if (act == DT_F32 && sketch == DT_F32) return launch_kda_f32(mode, coef, dk, dv, p, st);
  if (act == DT_BF16 && sketch == DT_BF16) return launch_dtype<FAM_KDA, bf16, bf16>(mode, coef, dk, dv, p, st);
  return -3;
}
}  // namespace sk
