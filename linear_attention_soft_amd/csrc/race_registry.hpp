// Registry of compiled kernel instances, keyed by (dtype, d, PE, LRP).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace race {

struct NCArgs;
struct WArgs;
struct TWArgs;
struct DArgs;
struct DWArgs;
struct Tables;

typedef void (*nc_launch_fn)(const NCArgs&, dim3 grid, hipStream_t);
typedef void (*tw_launch_fn)(const TWArgs&, dim3 grid, hipStream_t);
typedef void (*w_launch_fn)(const WArgs&, dim3 grid, hipStream_t);
typedef void (*dbg_launch_fn)(const void* X, const Tables& W, float beta, int L, int P, int64_t N, int dr,
                              float* out, dim3 grid, hipStream_t);

struct KernelSet {
  int dtype;   // race_dtype
  int D, PE, LRP;
  int NHP;     // hyperplane slots of the dPre rows: (LRP / 2^PE) * PE
  nc_launch_fn reduce;                     // bank / segment sums (both variants)
  nc_launch_fn readout, bwd_q, bwd_kv;     // non-causal; null when not compiled
  dbg_launch_fn softbucket_dbg;
  // causal; null when not compiled
  // causal walks (grid: segments x BH): readout layout, then transposed layout
  w_launch_fn w_segsum, w_gsum, w_fwd, w_h, w_dv;
  tw_launch_fn tw_dq, tw_dk;
  // the causal transposed walks read the projections W Q and W K that the
  // gradient-sum and dV walks store (split tables: 2^PE > 32)
  int tw_pre;
  // non-causal layer through static-bank walks (tables too wide for the
  // non-causal kernels' waves; the segment-sum walks come with them); null
  // when not compiled
  w_launch_fn w_fwd_st, w_h_st, w_dv_st;
  tw_launch_fn tw_dq_st, tw_dk_st;
  void (*h_from_o)(const void* dO, const void* O, const float* den, float* h, int64_t total, hipStream_t);
  // recurrent decode step (grid: BH)
  void (*decode)(const DArgs&, unsigned grid, hipStream_t);
  // table-gradient partials (grid: chunks x BH x 2 sides); null when the
  // set's dPre rows (NHP slots) are not a multiple of 4 floats
  void (*dw_partial)(const DWArgs&, dim3 grid, hipStream_t);
};

// Compiled kernel sets, one instance file per entry (race_inst_<name>.hip
// defines inst_<name>); the build lists exactly these files.
#define RACE_INSTANCE_FILES(X) \
  X(bf16_d64)                   \
  X(bf16_d128_p3)               \
  X(bf16_d128_p4)               \
  X(bf16_d128_p5)               \
  X(bf16_d128_p6)               \
  X(bf16_d128_p78)              \
  X(f32_d64)                    \
  X(f32_d128)

#define RACE_DECLARE_INSTANCE(name) const KernelSet* inst_##name(int* count);
RACE_INSTANCE_FILES(RACE_DECLARE_INSTANCE)
#undef RACE_DECLARE_INSTANCE

// Every compiled set, in instance-file order (built once, thread-safe).
const KernelSet* all_kernel_sets(int* count);

}  // namespace race
