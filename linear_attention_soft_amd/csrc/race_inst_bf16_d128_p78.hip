// Compiled kernel sets: bf16 I/O, head dim 128, P = 7 (128 corners per
// table, up to 2 tables) and P = 8 (256 corners, one table).  A table spans
// 4 or 8 waves of the transposed walks; the non-causal layer runs on the
// static-bank walks.  At P = 7 the dPre rows hold 14 slots per token, so the
// table gradient dW is not compiled there.
#include "race_inst.hpp"

namespace race {
const KernelSet* inst_bf16_d128_p78(int* count) {
  static const KernelSet sets[] = {
      Inst<bf16, 128, 7, 256>::template set<false, true, true>(1),
      Inst<bf16, 128, 8, 256>::template set<false, true, true>(1),
  };
  *count = (int)(sizeof(sets) / sizeof(sets[0]));
  return sets;
}
}  // namespace race
