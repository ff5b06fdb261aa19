// Compiled kernel instances for bf16 I/O.
#include "race_inst.hpp"

namespace race {
const KernelSet* kernel_sets_bf16(int* count) {
  static const KernelSet sets[] = {
      Inst<bf16, 64, 3, 32>::template set<true, false>(1),
      Inst<bf16, 64, 3, 128>::template set<false, true>(1),
      // the language-model shape keeps its 64-row bank: its forward walks
      // (inference) lose more to padding than its two transposed-walk waves
      // gain from it
      Inst<bf16, 64, 4, 64>::template set<true, true>(1),
      Inst<bf16, 128, 4, 32>::template set<true, false>(1),
      // causal walks at d = 128, P = 4 take a 128-row bank (zero rows past
      // L * 16): four transposed-walk waves of 32 rows instead of one wave
      // holding every dX column tile and spilling
      Inst<bf16, 128, 4, 128>::template set<false, true>(1),
      Inst<bf16, 128, 6, 256>::template set<false, true>(1),
  };
  *count = (int)(sizeof(sets) / sizeof(sets[0]));
  return sets;
}
}  // namespace race
