// Causal RACE attention (prefix bucket sums).  Host-side entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/race_attn.h"
#include "race_registry.hpp"

namespace race {

// Segments of the sequence processed by one workgroup each.
inline void causal_segmentation(int64_t N, int64_t BH, int* nseg, int64_t* seg_tokens) {
  int64_t want = (1024 + BH - 1) / BH;
  const int64_t tiles = (N + 63) / 64;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t per = (tiles + want - 1) / want;
  *seg_tokens = per * 64;
  *nseg = (int)((N + *seg_tokens - 1) / *seg_tokens);
}

inline race_status causal_forward(const KernelSet&, const void*, const void*, const void*, const float*, float, int,
                                  int, int64_t, int, int, int, int, int64_t, void*, void*, char*, hipStream_t,
                                  std::string* err) {
  *err = "causal kernels are not built";
  return RACE_ERR_UNSUPPORTED;
}

inline race_status causal_backward(const KernelSet&, const void*, const void*, const void*, const float*, float, int,
                                   int, int64_t, int, int, int, int, int64_t, const void*, void*, void*, void*,
                                   const void*, char*, hipStream_t, std::string* err) {
  *err = "causal kernels are not built";
  return RACE_ERR_UNSUPPORTED;
}

}  // namespace race
