// Compiled kernel sets: bf16 I/O, head dim 128, P <= 3 (tables widened to
// three hyperplanes): the (P, L) = (2, 2) and (3, 3) settings of the
// single-layer scaling runs.
#include "race_inst.hpp"

namespace race {
const KernelSet* inst_bf16_d128_p3(int* count) {
  static const KernelSet sets[] = {
      Inst<bf16, 128, 3, 32>::template set<true, false>(1),
      // causal walks take a 128-row bank (zero rows past L * 8), as at P = 4
      Inst<bf16, 128, 3, 128>::template set<false, true>(1),
  };
  *count = (int)(sizeof(sets) / sizeof(sets[0]));
  return sets;
}
}  // namespace race
