// Compiled kernel sets: bf16 I/O, head dim 128, P = 5 (32 corners per table,
// up to 4 tables).  The non-causal kernels' whole-bank LDS stages do not fit
// a 128-row bank at this table width, so the non-causal layer runs on the
// static-bank walks.
#include "race_inst.hpp"

namespace race {
const KernelSet* inst_bf16_d128_p5(int* count) {
  static const KernelSet sets[] = {
      Inst<bf16, 128, 5, 128>::template set<false, true, true>(1),
  };
  *count = (int)(sizeof(sets) / sizeof(sets[0]));
  return sets;
}
}  // namespace race
