// Compiled kernel sets: bf16 I/O, head dim 128, P = 6 (64 corners per table).
#include "race_inst.hpp"

namespace race {
const KernelSet* inst_bf16_d128_p6(int* count) {
  static const KernelSet sets[] = {
      Inst<bf16, 128, 6, 256>::template set<false, true, true>(1),
  };
  *count = (int)(sizeof(sets) / sizeof(sets[0]));
  return sets;
}
}  // namespace race
