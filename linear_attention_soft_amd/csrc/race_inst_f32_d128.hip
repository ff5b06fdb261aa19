// Compiled kernel sets: float32 I/O, head dim 128.
#include "race_inst.hpp"

namespace race {
const KernelSet* inst_f32_d128(int* count) {
  static const KernelSet sets[] = {
      Inst<float, 128, 3, 32>::template set<true, true>(0),
      Inst<float, 128, 4, 32>::template set<true, true>(0),
      // non-causal only: the causal transposed walk's float32 stages of a
      // 64-row bank need 169 KB of LDS, over the 160 KB of a CU
      Inst<float, 128, 4, 64>::template set<true, false>(0),
  };
  *count = (int)(sizeof(sets) / sizeof(sets[0]));
  return sets;
}
}  // namespace race
