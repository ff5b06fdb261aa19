// Compiled kernel sets: bf16 I/O, head dim 128, P = 4.
#include "race_inst.hpp"

namespace race {
const KernelSet* inst_bf16_d128_p4(int* count) {
  static const KernelSet sets[] = {
      Inst<bf16, 128, 4, 32>::template set<true, false>(1),
      // L = 3, 4: the (4, 4) setting of the single-layer scaling runs
      Inst<bf16, 128, 4, 64>::template set<true, false>(1),
      // causal walks at d = 128, P = 4 take a 128-row bank (zero rows past
      // L * 16): four transposed-walk waves of 32 rows instead of one wave
      // holding every dX column tile and spilling
      Inst<bf16, 128, 4, 128>::template set<false, true>(1),
  };
  *count = (int)(sizeof(sets) / sizeof(sets[0]));
  return sets;
}
}  // namespace race
