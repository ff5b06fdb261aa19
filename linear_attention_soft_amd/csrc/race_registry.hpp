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
typedef void (*dbg_launch_fn)(const void* X, const Tables& W, float beta, int L, int P, int64_t N,
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
  void (*h_from_o)(const void* dO, const void* O, const float* den, float* h, int64_t total, hipStream_t);
  // recurrent decode step (grid: BH)
  void (*decode)(const DArgs&, unsigned grid, hipStream_t);
  // table-gradient partials (grid: chunks x BH x 2 sides)
  void (*dw_partial)(const DWArgs&, dim3 grid, hipStream_t);
};

const KernelSet* kernel_sets_f32(int* count);
const KernelSet* kernel_sets_bf16(int* count);

}  // namespace race
