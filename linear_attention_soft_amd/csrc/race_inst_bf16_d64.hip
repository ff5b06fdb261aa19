// Compiled kernel sets: bf16 I/O, head dim 64.
#include "race_inst.hpp"

namespace race {
const KernelSet* inst_bf16_d64(int* count) {
  static const KernelSet sets[] = {
      Inst<bf16, 64, 3, 32>::template set<true, false>(1),
      Inst<bf16, 64, 3, 128>::template set<false, true>(1),
      // the language-model shape keeps its 64-row bank: its forward walks
      // (inference) lose more to padding than its two transposed-walk waves
      // gain from it
      Inst<bf16, 64, 4, 64>::template set<true, true>(1),
  };
  *count = (int)(sizeof(sets) / sizeof(sets[0]));
  return sets;
}
}  // namespace race
