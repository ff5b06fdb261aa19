// Compiled kernel instances for float32 I/O.
#include "race_inst.hpp"

namespace race {
const KernelSet* kernel_sets_f32(int* count) {
  static const KernelSet sets[] = {
      Inst<float, 64, 3, 32>::template set<true, true>(0),
      Inst<float, 64, 4, 64>::template set<true, true>(0),
      Inst<float, 128, 4, 32>::template set<true, true>(0),
  };
  *count = (int)(sizeof(sets) / sizeof(sets[0]));
  return sets;
}
}  // namespace race
