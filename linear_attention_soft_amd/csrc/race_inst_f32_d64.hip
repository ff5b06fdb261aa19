// Compiled kernel sets: float32 I/O, head dim 64.
#include "race_inst.hpp"

namespace race {
const KernelSet* inst_f32_d64(int* count) {
  static const KernelSet sets[] = {
      Inst<float, 64, 3, 32>::template set<true, true>(0),
      Inst<float, 64, 4, 64>::template set<true, true>(0),
  };
  *count = (int)(sizeof(sets) / sizeof(sets[0]));
  return sets;
}
}  // namespace race
