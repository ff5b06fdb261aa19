// C ABI of the RACE attention library: argument checks, size queries, kernel
// selection and launch.  Every check runs on the host before any work is
// enqueued; the library allocates no device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/race_attn.h"
#include "race_causal.hpp"
#include "race_noncausal.hpp"
#include "race_registry.hpp"
#include "race_walk.hpp"
#include "race_decode.hpp"
#include "race_dw.hpp"

namespace race {
// ------------------------------------------------------------------ fixed-order chunk sums
// bank[bh][lr][c] = sum over chunks of part[bh][chunk][lr][c] (c = d is the mass).
__global__ void race_bank_finalize(const float* __restrict__ part, int nchunk, int LRP, int D, int BH,
                                   float* __restrict__ content, float* __restrict__ mass) {
  const int64_t per = (int64_t)LRP * (D + 1);
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= per * BH) return;
  const int64_t bh = idx / per, rem = idx % per;
  const int lr = (int)(rem / (D + 1)), c = (int)(rem % (D + 1));
  const float* p = part + (size_t)bh * nchunk * per + rem;
  float s = 0.f;
  // unrolled so that several partial loads are in flight (the sum stays in chunk order)
#pragma unroll 8
  for (int k = 0; k < nchunk; ++k) s += p[(size_t)k * per];
  if (c < D) content[((size_t)bh * LRP + lr) * D + c] = s;
  else mass[(size_t)bh * LRP + lr] = s;
}

// Test export of banks in the pages' layout: out_c[b][l][r][c], out_m[b][l][r]
// for b < nbank, r < 2^P, from internal banks whose row of table l, corner
// r' is l * 2^PE + r'.  With P < 3 each corner r has 2^(PE - P) widened
// copies r' = r + e 2^P; they are summed back in a fixed order and scaled by
// copy_scale.  The zero hyperplanes split a key's assignment evenly over the
// copies, so a key bank's copies add up to the bank (scale 1); they also
// shrink Den by the same factor 2^(P - PE), so g and h grow by 2^(PE - P)
// and each copy of a gradient bank holds the whole gradient bank (scale
// 2^(P - PE)).  Content of bank b, row lr, column c sits at
// src_c[b * c_bank + lr * c_row + c], its mass at src_m[b * m_bank + lr * m_row].
__global__ void race_bank_export(const float* __restrict__ src_c, int64_t c_bank, int c_row,
                                 const float* __restrict__ src_m, int64_t m_bank, int m_row, int64_t nbank, int L,
                                 int P, int PE, int D, float copy_scale, float* __restrict__ out_c,
                                 float* __restrict__ out_m) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int R = 1 << P;
  const int64_t per = (int64_t)L * R * (D + 1);
  if (idx >= nbank * per) return;
  const int64_t b = idx / per, rem = idx % per;
  const int lr = (int)(rem / (D + 1)), c = (int)(rem % (D + 1));
  const int l = lr / R, r = lr % R;
  float s = 0.f;
  for (int e = 0; e < (1 << (PE - P)); ++e) {
    const int row = (l << PE) + r + (e << P);
    s += c < D ? src_c[b * c_bank + (int64_t)row * c_row + c] : src_m[b * m_bank + (int64_t)row * m_row];
  }
  s *= copy_scale;
  if (c < D) {
    if (out_c) out_c[(b * L * R + lr) * D + c] = s;
  } else if (out_m) {
    out_m[b * L * R + lr] = s;
  }
}

// Token rows copied between the caller's head dim and the kernels' (16-byte
// units): each destination row takes copy_w units from its source row and is
// zero past them.  Up to 8 tensors per launch (grid y); a NULL source skips.
struct RowCopies {
  const void* src[8];
  void* dst[8];
  int64_t rows;
  int src_w, dst_w, copy_w;
};
__global__ void race_copy_rows(RowCopies a) {
  const uint4* src = static_cast<const uint4*>(a.src[blockIdx.y]);
  uint4* dst = static_cast<uint4*>(a.dst[blockIdx.y]);
  if (!src) return;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= a.rows * a.dst_w) return;
  const int64_t r = idx / a.dst_w;
  const int c = (int)(idx % a.dst_w);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (c < a.copy_w) v = src[r * a.src_w + c];
  dst[r * a.dst_w + c] = v;
}

const KernelSet* all_kernel_sets(int* count) {
  static const std::vector<KernelSet> all = [] {
    std::vector<KernelSet> v;
    int n = 0;
#define RACE_COLLECT_INSTANCE(name)              \
  {                                              \
    const KernelSet* s = inst_##name(&n);        \
    v.insert(v.end(), s, s + n);                 \
  }
    RACE_INSTANCE_FILES(RACE_COLLECT_INSTANCE)
#undef RACE_COLLECT_INSTANCE
    return v;
  }();
  *count = (int)all.size();
  return all.data();
}

}  // namespace race

namespace {

thread_local std::string g_last_error;

// ---- optional kernel timing: HIP events recorded on the launch stream
struct ProfRec {
  hipEvent_t start, stop;
  const char* name;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct ProfScope {
  hipStream_t s;
  const char* name;
  hipEvent_t a = nullptr;
  ProfScope(hipStream_t st, const char* n) : s(st), name(n) {
    if (!g_prof_on) return;
    std::lock_guard<std::mutex> g(g_prof_mu);
    a = prof_event();
    if (a) (void)hipEventRecord(a, s);
  }
  ~ProfScope() {
    if (!a) return;
    std::lock_guard<std::mutex> g(g_prof_mu);
    hipEvent_t b = prof_event();
    if (!b) return;
    (void)hipEventRecord(b, s);
    g_prof_recs.push_back({a, b, name});
  }
};

race_status fail(race_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

struct Plan {
  int dtype = 0;
  int64_t B = 0, H = 0, N = 0, BH = 0;
  int64_t d = 0;   // the caller's head dim
  int64_t D = 0;   // the kernels' head dim (d rounded up to a compiled one; token rows padded when larger)
  int P = 0, L = 0, PE = 0, LR = 0, LRP = 0;
  bool causal = false;
  bool nc_static = false;    // non-causal layer through the static-bank walks
  bool w_per_head = false;   // W is [H][L][P][d] instead of [L][P][d]
  // non-causal chunking
  int nchunk = 0;
  int64_t chunk_tokens = 0;
  // causal segmentation
  int nseg = 0;
  int64_t seg_tokens = 0;
  const race::KernelSet* ks = nullptr;
};

size_t elem_size(int dtype) { return dtype == RACE_BF16 ? 2 : 4; }

const race::KernelSet* find_set(int dtype, int D, int PE, int LRP_min, bool causal) {
  int count = 0;
  const race::KernelSet* sets = race::all_kernel_sets(&count);
  const race::KernelSet* best = nullptr;
  for (int i = 0; i < count; ++i) {
    const race::KernelSet& k = sets[i];
    if (k.dtype != dtype || k.D != D || k.PE != PE || k.LRP < LRP_min) continue;
    if (causal && (!k.w_fwd || !k.tw_dq)) continue;
    if (!causal && !k.readout && !k.w_fwd_st) continue;
    // smallest padded bank; at equal size the non-causal kernels before the
    // static-bank walks
    if (!best || k.LRP < best->LRP || (k.LRP == best->LRP && !causal && k.readout && !best->readout)) best = &k;
  }
  return best;
}

void bind_set(Plan* p, const race::KernelSet* ks) {
  p->ks = ks;
  if (!ks) return;
  p->LRP = ks->LRP;
  p->nc_static = !p->causal && !ks->readout;
}

// Compiled head dims, smallest first: a caller's d runs on the smallest one at
// or above it that has a kernel set for (dtype, P, L, causal), its token rows
// padded with zero columns.
constexpr int kHeadDims[] = {64, 128};

void pick_set(Plan* p) {
  for (int D : kHeadDims) {
    if (D < p->d) continue;
    if (const race::KernelSet* ks = find_set(p->dtype, D, p->PE, p->LRP, p->causal)) {
      p->D = D;
      bind_set(p, ks);
      return;
    }
  }
  bind_set(p, nullptr);
}

// Decode and prefill need the bucket reduce and the decode kernel only (every
// compiled set has them); smallest padded bank first.
const race::KernelSet* find_decode_set(int dtype, int D, int PE, int LRP_min) {
  int count = 0;
  const race::KernelSet* sets = race::all_kernel_sets(&count);
  const race::KernelSet* best = nullptr;
  for (int i = 0; i < count; ++i) {
    const race::KernelSet& k = sets[i];
    if (k.dtype != dtype || k.D != D || k.PE != PE || k.LRP < LRP_min || !k.decode || !k.reduce) continue;
    if (!best || k.LRP < best->LRP) best = &k;
  }
  return best;
}

// Tokens per workgroup: at most about 1024 workgroups over the whole problem
// (several per compute unit on 256 CUs), at least one 128-token tile each;
// with min_tiles > 1, fewer workgroups of at least min_tiles tiles as long
// as every compute unit still gets one (about 256 workgroups).  Short
// sequences (the 64K-token classification shape) then fill a workgroup's
// tile pipeline and write fewer partial banks (at 2 x 4 x 64K tokens: 512
// workgroups of 8 tiles, Q- and K-side backward 0.065 / 0.068 -> 0.055 /
// 0.061 ms); long sequences keep 1024 workgroups.
constexpr int64_t kMinTilesPerWG = 8;
void chunking(int64_t N, int64_t BH, int64_t min_tiles, int* nchunk, int64_t* chunk_tokens) {
  const int64_t tiles = (N + race::TT - 1) / race::TT;
  int64_t want = (1024 + BH - 1) / BH;
  const int64_t fill = (256 + BH - 1) / BH;
  const int64_t deep = (tiles + min_tiles - 1) / min_tiles;
  const int64_t keep = deep > fill ? deep : fill;
  if (want > keep) want = keep;
  if (want < 1) want = 1;
  if (want > tiles) want = tiles;
  int64_t per_tiles = (tiles + want - 1) / want;
  *chunk_tokens = per_tiles * race::TT;
  *nchunk = (int)((N + *chunk_tokens - 1) / *chunk_tokens);
}

race_status make_plan(const race_shape* s, int P, int L, int causal, Plan* p, bool need_kernels) {
  if (!s) return fail(RACE_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 1 || s->H < 1 || s->N < 1 || s->d < 1)
    return fail(RACE_ERR_INVALID_ARG, "B, H, N and d must be >= 1");
  if (s->dtype != RACE_F32 && s->dtype != RACE_BF16) return fail(RACE_ERR_INVALID_ARG, "dtype must be RACE_F32 or RACE_BF16");
  if (s->w_per_head != 0 && s->w_per_head != 1) return fail(RACE_ERR_INVALID_ARG, "w_per_head must be 0 or 1");
  if (P < 1 || P > 8) return fail(RACE_ERR_INVALID_ARG, "P must be in [1, 8]");
  if (L < 1) return fail(RACE_ERR_INVALID_ARG, "L must be >= 1");
  if (causal != 0 && causal != 1) return fail(RACE_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (s->B > (int64_t)1 << 31 || s->H > (int64_t)1 << 31 || s->N > (int64_t)1 << 40 || s->d > 4096)
    return fail(RACE_ERR_INVALID_ARG, "shape out of range");
  p->dtype = s->dtype;
  p->B = s->B; p->H = s->H; p->N = s->N; p->d = s->d; p->BH = s->B * s->H;
  if (p->BH > 65535) return fail(RACE_ERR_UNSUPPORTED, "B*H above 65535 is not supported");
  p->P = P; p->L = L; p->PE = P < 3 ? 3 : P;
  if ((int64_t)L << p->PE > 256) return fail(RACE_ERR_UNSUPPORTED, "L * 2^max(P,3) above 256 is not supported");
  p->LR = L << p->PE;
  p->LRP = (p->LR + 31) / 32 * 32;
  p->causal = causal != 0;
  p->w_per_head = s->w_per_head != 0;
  if (p->d % 8 != 0 || p->d > 128) return fail(RACE_ERR_UNSUPPORTED, "head dim d must be a multiple of 8, at most 128");
  p->D = p->d <= 64 ? 64 : 128;
  if (need_kernels) {
    pick_set(p);
    if (!p->ks) return fail(RACE_ERR_UNSUPPORTED, "no compiled kernel for this (dtype, d, P, L, causal)");
  }
  chunking(p->N, p->BH, kMinTilesPerWG, &p->nchunk, &p->chunk_tokens);
  race::causal_segmentation(p->N, p->BH, &p->nseg, &p->seg_tokens);
  return RACE_OK;
}

// ---- sizes (bytes)
size_t bank_bytes(const Plan& p) { return (size_t)p.BH * p.LRP * (p.D + 1) * sizeof(float); }
size_t part_bytes(const Plan& p) { return (size_t)p.BH * p.nchunk * p.LRP * (p.D + 1) * sizeof(float); }
size_t seg_bank_bytes(const Plan& p) { return (size_t)p.BH * p.nseg * p.LRP * (p.D + 1) * sizeof(float); }
// Non-causal partial banks: one per chunk, or per segment (static-bank walks).
size_t nc_part_bytes(const Plan& p) { return p.nc_static ? seg_bank_bytes(p) : part_bytes(p); }
size_t tok_bytes(const Plan& p) { return (size_t)p.BH * p.N * sizeof(float); }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t state_bytes(const Plan& p) {
  if (!p.causal) return bank_bytes(p);
  return align256(seg_bank_bytes(p)) + align256(tok_bytes(p));
}


// Causal backward workspace: h [BH][N], gradient segment sums and their
// reverse scan [BH][nseg][LRP][d+1] each.
// Per-wave shares of dL/dbeta: query side then key side.  Non-causal: 4
// waves per (chunk, head); causal and static-bank walks: one wave per 32
// bucket rows per (segment, head) (the transposed walks' waves).
int64_t dbeta_parts_per_side(const Plan& p) {
  if (!p.causal && !p.nc_static) return (int64_t)p.BH * p.nchunk * 4;
  return (int64_t)p.BH * p.nseg * (p.LRP / 32);
}
size_t dbeta_bytes(const Plan& p) { return align256(2 * (size_t)dbeta_parts_per_side(p) * sizeof(float)); }

// Table gradient: dPre of both sides [2][BH][N][NHP] and the partials
// [2][BH][nchunk][NHP][d] of race_dw_partial.
int nhp(const Plan& p) { return p.ks ? p.ks->NHP : 0; }
size_t dpre_side_bytes(const Plan& p) { return align256((size_t)p.BH * p.N * nhp(p) * sizeof(float)); }

// Causal backward workspace: h, the gradient segment banks and their
// suffixes, dbeta shares, and (kernel sets whose transposed walks read them)
// the projections W Q and W K made once by the gradient-sum and dV walks for
// the walks after them (float32 [BH][N][NHP] each, the size of one dPre side).
struct CausalBwdWs {
  size_t h, gpart, gsuf, dbeta, preq, prek, total;
};
CausalBwdWs causal_bwd_ws(const Plan& p) {
  CausalBwdWs w{};
  size_t off = 0;
  w.h = off;     off += align256(tok_bytes(p));
  w.gpart = off; off += align256(seg_bank_bytes(p));
  w.gsuf = off;  off += align256(seg_bank_bytes(p));
  w.dbeta = off; off += dbeta_bytes(p);
  const size_t pre = (p.ks && p.ks->tw_pre) ? dpre_side_bytes(p) : 0;
  w.preq = off;  off += pre;
  w.prek = off;  off += pre;
  w.total = off;
  return w;
}

// dW partials [2][BH][nchunk][NHP][d] of race_dw_partial (after the dPre
// rows of both sides).
size_t dw_part_bytes(const Plan& p) {
  return align256(2 * (size_t)p.BH * p.nchunk * nhp(p) * p.D * sizeof(float));
}
size_t dw_bytes(const Plan& p) { return 2 * dpre_side_bytes(p) + dw_part_bytes(p); }
size_t dw_out_floats(const Plan& p) { return (size_t)(p.w_per_head ? p.H : 1) * p.L * p.P * p.d; }

// Bytes of the state a backward rebuilds itself when the caller passes none
// (non-causal: the bank; causal: segment banks and Den; the causal segment
// sums go to the backward's own gradient-sum region first).
size_t rebuilt_state_bytes(const Plan& p) { return p.causal ? state_bytes(p) : align256(bank_bytes(p)); }

// Workspace layout: the phase's own scratch, then (backward with dW) the
// table-gradient region, then (backward without a state) the rebuilt state.
size_t workspace_bytes(const Plan& p, bool bwd, bool dw = false, bool no_state = false) {
  if (bwd && no_state) return workspace_bytes(p, true, dw, false) + rebuilt_state_bytes(p);
  if (bwd && dw) return workspace_bytes(p, true, false) + dw_bytes(p);
  if (!p.causal) {
    size_t w = align256(nc_part_bytes(p));
    if (!bwd) return w + align256(bank_bytes(p));   // bank when no state buffer is given
    w += align256(bank_bytes(p)) + dbeta_bytes(p);  // gradient bank dcontent, dmass; dbeta shares
    if (p.nc_static) w += 2 * align256(tok_bytes(p));   // h and Den of every query
    return w;
  }
  // forward: segment sums, and (when no state buffer is given) the segment
  // banks and Den
  if (!bwd) return align256(seg_bank_bytes(p)) + align256(seg_bank_bytes(p)) + align256(tok_bytes(p));
  return causal_bwd_ws(p).total;
}

// When the caller's head dim d is below the kernels' D, the entry points
// work on zero-padded copies of the token tensors, appended to the
// workspace: forward Q, K, V, O (4), backward Q, K, V, dO, O, dQ, dK, dV (8),
// prefill K, V (2).
size_t padded_tensor_bytes(const Plan& p) { return align256((size_t)p.BH * p.N * p.D * elem_size(p.dtype)); }
size_t pad_bytes(const Plan& p, int tensors) { return p.d == p.D ? 0 : (size_t)tensors * padded_tensor_bytes(p); }
size_t total_workspace_bytes(const Plan& p, bool bwd, bool dw = false, bool no_state = false) {
  return workspace_bytes(p, bwd, dw, no_state) + pad_bytes(p, bwd ? 8 : 4);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b) return false;
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

race_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RACE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return RACE_OK;
}

// Copies n token tensors [BH][N][row] between the caller's head dim and the
// kernels' (to_kernel: caller -> zero-padded kernel rows; else back).
race_status copy_rows(const Plan& p, const void* const* src, void* const* dst, int n, bool to_kernel, hipStream_t s) {
  race::RowCopies a{};
  for (int i = 0; i < n; ++i) { a.src[i] = src[i]; a.dst[i] = dst[i]; }
  const int cw = (int)(p.d * (int64_t)elem_size(p.dtype) / 16), kw = (int)(p.D * (int64_t)elem_size(p.dtype) / 16);
  a.rows = p.BH * p.N;
  a.src_w = to_kernel ? cw : kw;
  a.dst_w = to_kernel ? kw : cw;
  a.copy_w = cw;
  const int64_t blocks = (a.rows * a.dst_w + 255) / 256;
  {
    ProfScope ps(s, "race_copy_rows");
    hipLaunchKernelGGL(race::race_copy_rows, dim3((unsigned)blocks, (unsigned)n), dim3(256), 0, s, a);
  }
  return check_launch("race_copy_rows");
}

void launch_finalize(const float* part, int nchunk, const Plan& p, float* content, float* mass, hipStream_t st) {
  const int64_t total = p.BH * (int64_t)p.LRP * (p.D + 1);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(race::race_bank_finalize, dim3((unsigned)blocks), dim3(threads), 0, st, part, nchunk,
                     p.LRP, (int)p.D, (int)p.BH, content, mass);
}


// ---- causal sequences
race::Tables tables(const Plan& p, const float* W) {
  race::Tables t;
  t.W = W;
  t.hstride = p.w_per_head ? (int64_t)p.L * p.P * p.d : 0;
  t.ld = (int)p.d;
  t.H = (int)p.H;
  return t;
}

race::WArgs walk_args(const Plan& p, const float* W, float beta) {
  race::WArgs w{};
  w.W = tables(p, W); w.beta = beta; w.L = p.L; w.P = p.P; w.N = p.N; w.seg_tokens = p.seg_tokens; w.nseg = p.nseg;
  return w;
}

void launch_dbeta_finalize(const Plan& p, const float* parts, float* dbeta, hipStream_t s) {
  hipLaunchKernelGGL(race::race_dbeta_finalize, dim3(1), dim3(256), 0, s, parts, 2 * dbeta_parts_per_side(p), dbeta);
}

// dW from the dPre rows the backward kernels wrote into the workspace's
// table-gradient region (query side, key side, partials).
race_status launch_dw(const Plan& p, const void* Q, const void* K, float* dW, char* region, hipStream_t s) {
  race_status st;
  race::DWArgs a{};
  a.X0 = Q; a.X1 = K;
  a.dpre0 = reinterpret_cast<const float*>(region);
  a.dpre1 = reinterpret_cast<const float*>(region + dpre_side_bytes(p));
  a.part = reinterpret_cast<float*>(region + 2 * dpre_side_bytes(p));
  a.N = p.N; a.chunk_tokens = p.chunk_tokens; a.nchunk = p.nchunk;
  {
    ProfScope ps(s, "race_dw_partial");
    p.ks->dw_partial(a, dim3((unsigned)p.nchunk, (unsigned)p.BH, 2), s);
  }
  if ((st = check_launch("race_dw_partial")) != RACE_OK) return st;
  const unsigned rows = (unsigned)((p.w_per_head ? p.H : 1) * p.L * p.P);
  {
    ProfScope ps(s, "race_dw_finalize");
    hipLaunchKernelGGL(race::race_dw_finalize, dim3(rows), dim3(1024), 0, s, a.part, (int)p.B, (int)p.H,
                       p.w_per_head ? 1 : 0, p.nchunk, nhp(p), p.PE, p.L, p.P, (int)p.D, (int)p.d, dW);
  }
  return check_launch("race_dw_finalize");
}

void launch_seg_scan(const Plan& p, const float* part, float* out, int reverse, hipStream_t s) {
  const int per = p.LRP * (int)(p.D + 1);
  const int64_t tot = p.BH * (int64_t)per;
  hipLaunchKernelGGL(race::race_seg_scan, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, part, out, p.nseg,
                     per, (int)p.BH, reverse);
}

// Segment sums into part, their exclusive scan into prefix, then the forward
// walk: O (skipped when NULL) and Den.
race_status causal_forward_into(const Plan& p, const void* Q, const void* K, const void* V, const float* W, float beta,
                                void* O, float* part, float* prefix, float* den, hipStream_t s) {
  race_status st;
  const dim3 grid((unsigned)p.nseg, (unsigned)p.BH);
  race::WArgs w = walk_args(p, W, beta);
  w.B_src = K; w.X_src = V; w.bank_out = part;
  {
    ProfScope ps(s, "race_causal_segsum");
    p.ks->w_segsum(w, grid, s);
  }
  if ((st = check_launch("race_causal_segsum")) != RACE_OK) return st;
  {
    ProfScope ps(s, "race_seg_scan");
    launch_seg_scan(p, part, prefix, 0, s);
  }
  if ((st = check_launch("race_seg_scan")) != RACE_OK) return st;
  w = walk_args(p, W, beta);
  w.A_src = Q; w.B_src = K; w.X_src = V; w.out = O; w.bank_in = prefix; w.den_out = den;
  {
    ProfScope ps(s, "race_causal_fwd");
    p.ks->w_fwd(w, grid, s);
  }
  return check_launch("race_causal_fwd");
}

race_status causal_forward(const Plan& p, const void* Q, const void* K, const void* V, const float* W, float beta,
                           void* O, void* state, char* ws, hipStream_t s) {
  float* part = reinterpret_cast<float*>(ws);
  char* sbase = state ? static_cast<char*>(state) : ws + align256(seg_bank_bytes(p));
  float* prefix = reinterpret_cast<float*>(sbase);
  float* den = reinterpret_cast<float*>(sbase + align256(seg_bank_bytes(p)));
  return causal_forward_into(p, Q, K, V, W, beta, O, part, prefix, den, s);
}

// Non-causal bank of K, V: partial banks into part, fixed-order sums into
// content / mass.
race_status noncausal_bank(const Plan& p, const void* K, const void* V, const float* W, float beta, float* part,
                           float* content, float* mass, hipStream_t s) {
  race_status st;
  if (p.nc_static) {
    // segment sums from the segment-sum walk, then their fixed-order sum
    race::WArgs w = walk_args(p, W, beta);
    w.B_src = K; w.X_src = V; w.bank_out = part;
    {
      ProfScope ps(s, "race_causal_segsum");
      p.ks->w_segsum(w, dim3((unsigned)p.nseg, (unsigned)p.BH), s);
    }
    if ((st = check_launch("race_causal_segsum")) != RACE_OK) return st;
    {
      ProfScope ps(s, "race_bank_finalize");
      launch_finalize(part, p.nseg, p, content, mass, s);
    }
    return check_launch("race_bank_finalize");
  }
  race::NCArgs a{};
  a.X = K; a.Y = V; a.W = tables(p, W); a.beta = beta; a.L = p.L; a.P = p.P; a.N = p.N;
  a.chunk_tokens = p.chunk_tokens; a.nchunk = p.nchunk; a.part = part;
  {
    ProfScope ps(s, "race_bucket_reduce");
    p.ks->reduce(a, dim3(p.nchunk, (unsigned)p.BH), s);
  }
  if ((st = check_launch("race_bucket_reduce")) != RACE_OK) return st;
  {
    ProfScope ps(s, "race_bank_finalize");
    launch_finalize(part, p.nchunk, p, content, mass, s);
  }
  return check_launch("race_bank_finalize");
}

race_status causal_backward(const Plan& p, const void* Q, const void* K, const void* V, const float* W, float beta,
                            const void* O, const void* dO, void* dQ, void* dK, void* dV, float* dbeta,
                            float* dW, const void* state, char* ws, hipStream_t s) {
  race_status st;
  const float* prefix = static_cast<const float*>(state);
  const float* den = reinterpret_cast<const float*>(static_cast<const char*>(state) + align256(seg_bank_bytes(p)));
  const CausalBwdWs L = causal_bwd_ws(p);
  float* h = reinterpret_cast<float*>(ws + L.h);
  float* gpart = reinterpret_cast<float*>(ws + L.gpart);
  float* gsuf = reinterpret_cast<float*>(ws + L.gsuf);
  float* preq = p.ks->tw_pre ? reinterpret_cast<float*>(ws + L.preq) : nullptr;
  float* prek = p.ks->tw_pre ? reinterpret_cast<float*>(ws + L.prek) : nullptr;
  const dim3 grid((unsigned)p.nseg, (unsigned)p.BH);

  // 1. h = -(dO . O) / Den: elementwise from O when the caller has it, else
  //    from a readout walk that rebuilds Den O without writing O
  race::WArgs w = walk_args(p, W, beta);
  if (O) {
    ProfScope ps(s, "race_causal_h_from_o");
    p.ks->h_from_o(dO, O, den, h, p.BH * p.N, s);
  } else {
    w.A_src = Q; w.B_src = K; w.X_src = V; w.dO = dO; w.bank_in = prefix; w.den = den; w.h_out = h;
    ProfScope ps(s, "race_causal_h");
    p.ks->w_h(w, grid, s);
  }
  if ((st = check_launch("race_causal_h")) != RACE_OK) return st;
  // 2. gradient segment sums Phi_Q^T [g | h], reverse exclusive scan; the
  //    walk keeps its projections W Q for the walks below
  w = walk_args(p, W, beta);
  w.B_src = Q; w.X_src = dO; w.den = den; w.hvec = h; w.bank_out = gpart; w.pre_out = preq;
  {
    ProfScope ps(s, "race_causal_gradsum");
    p.ks->w_gsum(w, grid, s);
  }
  if ((st = check_launch("race_causal_gradsum")) != RACE_OK) return st;
  launch_seg_scan(p, gpart, gsuf, 1, s);
  if ((st = check_launch("race_seg_scan")) != RACE_OK) return st;
  // 3. dV: reverse walk with Phi_K as output role, Phi_Q as state role (from
  //    the stored W Q where kept), g as values; it keeps its projections W K
  w = walk_args(p, W, beta);
  w.A_src = K; w.B_src = Q; w.X_src = dO; w.den = den; w.bank_in = gsuf; w.out = dV; w.pre_out = prek;
  w.preB_in = preq;
  {
    ProfScope ps(s, "race_causal_dv");
    p.ks->w_dv(w, grid, s);
  }
  if ((st = check_launch("race_causal_dv")) != RACE_OK) return st;
  // 4. dQ: forward transposed walk (dPhi_Q, softmax / tanh / projection backward)
  race::TWArgs t{};
  t.W = tables(p, W); t.beta = beta; t.L = p.L; t.P = p.P; t.N = p.N; t.seg_tokens = p.seg_tokens; t.nseg = p.nseg;
  t.den = den; t.hvec = h;
  float* bparts = dbeta ? reinterpret_cast<float*>(ws + L.dbeta) : nullptr;
  char* dwr = dW ? ws + L.total : nullptr;
  t.A_src = Q; t.B_src = K; t.X_src = V; t.U_src = dO; t.bank_in = prefix; t.dX = dQ; t.dbeta_part = bparts;
  t.preA_in = preq; t.preB_in = prek;
  t.dpre_out = dwr ? reinterpret_cast<float*>(dwr) : nullptr;
  {
    ProfScope ps(s, "race_causal_dq");
    p.ks->tw_dq(t, grid, s);
  }
  if ((st = check_launch("race_causal_dq")) != RACE_OK) return st;
  // 5. dK: reverse transposed walk (dPhi_K) from the gradient suffix banks
  t.A_src = K; t.B_src = Q; t.X_src = dO; t.U_src = V; t.bank_in = gsuf; t.dX = dK;
  t.preA_in = prek; t.preB_in = preq;
  t.dbeta_part = bparts ? bparts + dbeta_parts_per_side(p) : nullptr;
  t.dpre_out = dwr ? reinterpret_cast<float*>(dwr + dpre_side_bytes(p)) : nullptr;
  {
    ProfScope ps(s, "race_causal_dk");
    p.ks->tw_dk(t, grid, s);
  }
  if ((st = check_launch("race_causal_dk")) != RACE_OK) return st;
  if (dbeta) {
    ProfScope ps(s, "race_dbeta_finalize");
    launch_dbeta_finalize(p, bparts, dbeta, s);
  }
  if ((st = check_launch("race_dbeta_finalize")) != RACE_OK) return st;
  return dW ? launch_dw(p, Q, K, dW, dwr, s) : RACE_OK;
}

// Non-causal backward through the static-bank walks: Den and h from a
// readout of the bank, the gradient bank as segment sums of Phi_Q^T [g | h]
// and their fixed-order sum, then dV = Phi_K dcontent and the transposed
// walks for dQ (bank of K, V) and dK (gradient bank).
race_status static_backward(const Plan& p, const void* Q, const void* K, const void* V, const float* W, float beta,
                            const void* dO, void* dQ, void* dK, void* dV, float* dbeta, float* dW,
                            const void* state, char* ws, hipStream_t s) {
  race_status st;
  const float* content = static_cast<const float*>(state);
  const float* mass = content + (size_t)p.BH * p.LRP * p.D;
  float* part = reinterpret_cast<float*>(ws);
  char* after_part = ws + align256(nc_part_bytes(p));
  float* dcontent = reinterpret_cast<float*>(after_part);
  float* dmass = dcontent + (size_t)p.BH * p.LRP * p.D;
  char* after_bank = after_part + align256(bank_bytes(p));
  float* bparts = dbeta ? reinterpret_cast<float*>(after_bank) : nullptr;
  float* h = reinterpret_cast<float*>(after_bank + dbeta_bytes(p));
  float* den = reinterpret_cast<float*>(after_bank + dbeta_bytes(p) + align256(tok_bytes(p)));
  char* dwr = dW ? ws + workspace_bytes(p, true, false) : nullptr;
  const dim3 grid((unsigned)p.nseg, (unsigned)p.BH);

  // 1. Den and h = -(dO . Phi_Q content) / Den^2 of every query
  race::WArgs w = walk_args(p, W, beta);
  w.A_src = Q; w.dO = dO; w.bank_in = content; w.mass_in = mass; w.h_out = h; w.den_out = den;
  {
    ProfScope ps(s, "race_static_h");
    p.ks->w_h_st(w, grid, s);
  }
  if ((st = check_launch("race_static_h")) != RACE_OK) return st;
  // 2. gradient bank: segment sums of Phi_Q^T [g | h], summed in segment order
  w = walk_args(p, W, beta);
  w.B_src = Q; w.X_src = dO; w.den = den; w.hvec = h; w.bank_out = part;
  {
    ProfScope ps(s, "race_causal_gradsum");
    p.ks->w_gsum(w, grid, s);
  }
  if ((st = check_launch("race_causal_gradsum")) != RACE_OK) return st;
  {
    ProfScope ps(s, "race_bank_finalize");
    launch_finalize(part, p.nseg, p, dcontent, dmass, s);
  }
  if ((st = check_launch("race_bank_finalize")) != RACE_OK) return st;
  // 3. dV = Phi_K dcontent
  w = walk_args(p, W, beta);
  w.A_src = K; w.bank_in = dcontent; w.mass_in = dmass; w.out = dV;
  {
    ProfScope ps(s, "race_static_dv");
    p.ks->w_dv_st(w, grid, s);
  }
  if ((st = check_launch("race_static_dv")) != RACE_OK) return st;
  // 4. dQ, dK: transposed walks against the fixed banks
  race::TWArgs t{};
  t.W = tables(p, W); t.beta = beta; t.L = p.L; t.P = p.P; t.N = p.N; t.seg_tokens = p.seg_tokens; t.nseg = p.nseg;
  t.den = den; t.hvec = h;
  t.A_src = Q; t.U_src = dO; t.bank_in = content; t.mass_in = mass; t.dX = dQ; t.dbeta_part = bparts;
  t.dpre_out = dwr ? reinterpret_cast<float*>(dwr) : nullptr;
  {
    ProfScope ps(s, "race_static_dq");
    p.ks->tw_dq_st(t, grid, s);
  }
  if ((st = check_launch("race_static_dq")) != RACE_OK) return st;
  t.A_src = K; t.U_src = V; t.bank_in = dcontent; t.mass_in = dmass; t.dX = dK;
  t.dbeta_part = bparts ? bparts + dbeta_parts_per_side(p) : nullptr;
  t.dpre_out = dwr ? reinterpret_cast<float*>(dwr + dpre_side_bytes(p)) : nullptr;
  {
    ProfScope ps(s, "race_static_dk");
    p.ks->tw_dk_st(t, grid, s);
  }
  if ((st = check_launch("race_static_dk")) != RACE_OK) return st;
  if (dbeta) {
    ProfScope ps(s, "race_dbeta_finalize");
    launch_dbeta_finalize(p, bparts, dbeta, s);
  }
  if ((st = check_launch("race_dbeta_finalize")) != RACE_OK) return st;
  return dW ? launch_dw(p, Q, K, dW, dwr, s) : RACE_OK;
}

}  // namespace

extern "C" {

size_t race_attn_state_bytes(const race_shape* shape, int P, int L, int causal) {
  Plan p;
  if (make_plan(shape, P, L, causal, &p, false) != RACE_OK) return 0;
  pick_set(&p);
  return state_bytes(p);
}

size_t race_attn_workspace_bytes(const race_shape* shape, int P, int L, int causal, int is_bwd) {
  Plan p;
  const int phase = is_bwd & ~RACE_WS_NO_STATE;
  const bool no_state = (is_bwd & RACE_WS_NO_STATE) != 0;
  if (phase < RACE_WS_FWD || phase > RACE_WS_BWD_DW || (no_state && phase == RACE_WS_FWD)) return 0;
  if (make_plan(shape, P, L, causal, &p, false) != RACE_OK) return 0;
  pick_set(&p);
  return total_workspace_bytes(p, phase != RACE_WS_FWD, phase == RACE_WS_BWD_DW, no_state);
}

}  // extern "C"

namespace {

// ---- scratch of the allocation-free forward: one copy per GPU, held by
// the code object until the process ends.  In host code the name `scratch`
// is only a stand-in for the symbol; every use goes through the device
// address that hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device ordinal; null until looked up

race_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RACE_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(RACE_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return RACE_OK;
}

// Workspace the forward touches: the partial banks (non-causal) or segment
// sums (causal), plus the state's own room when the caller passes no state.
size_t fwd_workspace_used(const Plan& p, bool have_state) {
  if (have_state) return (p.causal ? align256(seg_bank_bytes(p)) : align256(nc_part_bytes(p))) + pad_bytes(p, 4);
  return total_workspace_bytes(p, false);
}

// The backward on token tensors of the kernels' head dim: the state rebuilt
// first when the caller passes none, then the variant's kernels.
race_status bwd_run(const Plan& p, const void* Q, const void* K, const void* V, const float* W, float beta,
                    const void* O, const void* dO, void* dQ, void* dK, void* dV, float* dbeta, float* dW,
                    const void* state, char* ws, hipStream_t s) {
  race_status st;
  if (!state) {
    // rebuild the forward's state at the end of the workspace: the bank of K,
    // V (non-causal), or the segment banks and Den (causal; O is not written)
    char* sreg = ws + workspace_bytes(p, true, dW != nullptr, false);
    if (p.causal) {
      float* gpart = reinterpret_cast<float*>(ws + causal_bwd_ws(p).gpart);
      float* prefix = reinterpret_cast<float*>(sreg);
      float* den = reinterpret_cast<float*>(sreg + align256(seg_bank_bytes(p)));
      st = causal_forward_into(p, Q, K, V, W, beta, nullptr, gpart, prefix, den, s);
    } else {
      float* content = reinterpret_cast<float*>(sreg);
      st = noncausal_bank(p, K, V, W, beta, reinterpret_cast<float*>(ws), content,
                          content + (size_t)p.BH * p.LRP * p.D, s);
    }
    if (st != RACE_OK) return st;
    state = sreg;
  }
  if (p.causal) return causal_backward(p, Q, K, V, W, beta, O, dO, dQ, dK, dV, dbeta, dW, state, ws, s);
  if (p.nc_static) return static_backward(p, Q, K, V, W, beta, dO, dQ, dK, dV, dbeta, dW, state, ws, s);
  char* dwr = dW ? ws + workspace_bytes(p, true, false) : nullptr;

  const float* content = static_cast<const float*>(state);
  const float* mass = content + (size_t)p.BH * p.LRP * p.D;
  float* part = reinterpret_cast<float*>(ws);
  float* dbank = reinterpret_cast<float*>(ws + align256(part_bytes(p)));
  float* dcontent = dbank;
  float* dmass = dbank + (size_t)p.BH * p.LRP * p.D;
  float* bparts = dbeta ? reinterpret_cast<float*>(ws + align256(part_bytes(p)) + align256(bank_bytes(p))) : nullptr;

  race::NCArgs a{};
  a.X = Q; a.Y = dO; a.out0 = dQ; a.W = tables(p, W); a.beta = beta; a.L = p.L; a.P = p.P; a.N = p.N;
  a.st_content = content; a.st_mass = mass; a.part = part;
  a.chunk_tokens = p.chunk_tokens; a.nchunk = p.nchunk; a.dbeta_part = bparts;
  a.dpre_out = dwr ? reinterpret_cast<float*>(dwr) : nullptr;
  {
    ProfScope ps(s, "race_bwd_q");
    p.ks->bwd_q(a, dim3(p.nchunk, (unsigned)p.BH), s);
  }
  if ((st = check_launch("race_bwd_q")) != RACE_OK) return st;
  {
    ProfScope ps(s, "race_bank_finalize");
    launch_finalize(part, p.nchunk, p, dcontent, dmass, s);
  }
  if ((st = check_launch("race_bank_finalize")) != RACE_OK) return st;
  race::NCArgs b{};
  b.X = K; b.Y = V; b.out0 = dV; b.out1 = dK; b.W = tables(p, W); b.beta = beta; b.L = p.L; b.P = p.P; b.N = p.N;
  b.st_content = dcontent; b.st_mass = dmass; b.chunk_tokens = p.chunk_tokens; b.nchunk = p.nchunk;
  b.dbeta_part = bparts ? bparts + dbeta_parts_per_side(p) : nullptr;
  b.dpre_out = dwr ? reinterpret_cast<float*>(dwr + dpre_side_bytes(p)) : nullptr;
  {
    ProfScope ps(s, "race_bwd_kv");
    p.ks->bwd_kv(b, dim3(p.nchunk, (unsigned)p.BH), s);
  }
  if ((st = check_launch("race_bwd_kv")) != RACE_OK) return st;
  if (dbeta) {
    ProfScope ps(s, "race_dbeta_finalize");
    launch_dbeta_finalize(p, bparts, dbeta, s);
  }
  if ((st = check_launch("race_dbeta_finalize")) != RACE_OK) return st;
  return dW ? launch_dw(p, Q, K, dW, dwr, s) : RACE_OK;
}

race_status fwd_run(const Plan& p, const void* Q, const void* K, const void* V, const float* W, float beta, void* O,
                    void* state, char* ws, hipStream_t s);

// Shared by race_attn_fwd (caller's workspace, at least the documented
// race_attn_workspace_bytes) and race_attn_fwd_noalloc (the library's own
// scratch, at least what this call touches).
race_status fwd_common(const void* Q, const void* K, const void* V, const float* W, float beta, int P, int L,
                       int causal, void* O, const race_shape* shape, void* state, size_t state_bytes_in,
                       void* workspace, size_t workspace_bytes_in, race_stream_t stream, bool own_scratch) {
  g_last_error.clear();
  Plan p;
  race_status st = make_plan(shape, P, L, causal, &p, true);
  if (st != RACE_OK) return st;
  if (!Q || !K || !V || !W || !O) return fail(RACE_ERR_INVALID_ARG, "Q, K, V, W and O must be non-NULL");
  if (!std::isfinite(beta)) return fail(RACE_ERR_INVALID_ARG, "beta must be finite");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(W) ||
      (state && !aligned16(state)) || (workspace && !aligned16(workspace)))
    return fail(RACE_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  const size_t tbytes = (size_t)(p.BH * p.N * p.d) * elem_size(p.dtype);
  if (overlaps(O, tbytes, Q, tbytes) || overlaps(O, tbytes, K, tbytes) || overlaps(O, tbytes, V, tbytes))
    return fail(RACE_ERR_INVALID_ARG, "O overlaps an input");
  if (own_scratch) {
    const size_t used = fwd_workspace_used(p, state != nullptr);
    if (used > workspace_bytes_in)
      return fail(RACE_ERR_WORKSPACE, "this call needs " + std::to_string(used) +
                                          " bytes of scratch, above the " + std::to_string(workspace_bytes_in) +
                                          " bytes the allocation-free forward holds");
  } else {
    const size_t need_ws = total_workspace_bytes(p, false);
    if (!workspace || workspace_bytes_in < need_ws)
      return fail(RACE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need_ws) + " bytes");
  }
  const size_t need_ws = own_scratch ? 0 : total_workspace_bytes(p, false);
  const size_t need_state = state_bytes(p);
  if (state && state_bytes_in < need_state)
    return fail(RACE_ERR_WORKSPACE, "state too small: need " + std::to_string(need_state) + " bytes");
  if (state && (overlaps(state, need_state, O, tbytes) || overlaps(state, need_state, workspace, need_ws)))
    return fail(RACE_ERR_INVALID_ARG, "state overlaps O or the workspace");
  if (own_scratch) {
    // every argument check has passed: look up this device's scratch
    if ((st = scratch_address(&workspace)) != RACE_OK) return st;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (p.d == p.D) return fwd_run(p, Q, K, V, W, beta, O, state, ws, s);
  // the caller's head dim is below the kernels': zero-padded copies of Q, K,
  // V and O after the forward's own workspace
  char* r = ws + fwd_workspace_used(p, state != nullptr) - pad_bytes(p, 4);
  const size_t tb = padded_tensor_bytes(p);
  void* kt[4] = {r, r + tb, r + 2 * tb, r + 3 * tb};
  const void* src[] = {Q, K, V};
  if ((st = copy_rows(p, src, kt, 3, true, s)) != RACE_OK) return st;
  if ((st = fwd_run(p, kt[0], kt[1], kt[2], W, beta, kt[3], state, ws, s)) != RACE_OK) return st;
  const void* res[] = {kt[3]};
  void* out[] = {O};
  return copy_rows(p, res, out, 1, false, s);
}

// The forward on token tensors of the kernels' head dim.
race_status fwd_run(const Plan& p, const void* Q, const void* K, const void* V, const float* W, float beta, void* O,
                    void* state, char* ws, hipStream_t s) {
  race_status st;
  if (p.causal) return causal_forward(p, Q, K, V, W, beta, O, state, ws, s);

  float* part = reinterpret_cast<float*>(ws);
  float* bank = state ? static_cast<float*>(state) : reinterpret_cast<float*>(ws + align256(nc_part_bytes(p)));
  float* content = bank;
  float* mass = bank + (size_t)p.BH * p.LRP * p.D;
  if ((st = noncausal_bank(p, K, V, W, beta, part, content, mass, s)) != RACE_OK) return st;
  if (p.nc_static) {
    race::WArgs w = walk_args(p, W, beta);
    w.A_src = Q; w.out = O; w.bank_in = content; w.mass_in = mass;
    {
      ProfScope ps(s, "race_static_fwd");
      p.ks->w_fwd_st(w, dim3((unsigned)p.nseg, (unsigned)p.BH), s);
    }
    return check_launch("race_static_fwd");
  }
  race::NCArgs r{};
  r.X = Q; r.out0 = O; r.W = tables(p, W); r.beta = beta; r.L = p.L; r.P = p.P; r.N = p.N;
  r.st_content = content; r.st_mass = mass; r.chunk_tokens = p.chunk_tokens; r.nchunk = p.nchunk;
  {
    ProfScope ps(s, "race_readout_norm");
    p.ks->readout(r, dim3(p.nchunk, (unsigned)p.BH), s);
  }
  return check_launch("race_readout_norm");
}

}  // namespace

extern "C" {

race_status race_attn_fwd(const void* Q, const void* K, const void* V, const float* W, float beta, int P, int L,
                          int causal, void* O, const race_shape* shape, void* state, size_t state_bytes_in,
                          void* workspace, size_t workspace_bytes_in, race_stream_t stream) {
  return fwd_common(Q, K, V, W, beta, P, L, causal, O, shape, state, state_bytes_in, workspace, workspace_bytes_in,
                    stream, false);
}

size_t race_attn_fwd_noalloc_scratch_bytes(void) { return kScratchBytes; }

race_status race_attn_fwd_noalloc(const void* Q, const void* K, const void* V, const float* W, float beta, int P,
                                  int L, int causal, void* O, const race_shape* shape, void* state,
                                  size_t state_bytes_in, race_stream_t stream) {
  return fwd_common(Q, K, V, W, beta, P, L, causal, O, shape, state, state_bytes_in, nullptr, kScratchBytes, stream,
                    true);
}

race_status race_attn_bwd(const void* Q, const void* K, const void* V, const float* W, float beta, int P, int L,
                          int causal, const void* O, const void* dO, void* dQ, void* dK, void* dV, float* dbeta,
                          float* dW, const race_shape* shape, const void* state, size_t state_bytes_in, void* workspace,
                          size_t workspace_bytes_in, race_stream_t stream) {
  g_last_error.clear();
  Plan p;
  race_status st = make_plan(shape, P, L, causal, &p, true);
  if (st != RACE_OK) return st;
  if (!Q || !K || !V || !W || !dO || !dQ || !dK || !dV)
    return fail(RACE_ERR_INVALID_ARG, "Q, K, V, W, dO, dQ, dK and dV must be non-NULL");
  if (!std::isfinite(beta)) return fail(RACE_ERR_INVALID_ARG, "beta must be finite");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(W) || !aligned16(dO) || !aligned16(dQ) ||
      !aligned16(dK) || !aligned16(dV) || (state && !aligned16(state)) || (O && !aligned16(O)) ||
      (workspace && !aligned16(workspace)))
    return fail(RACE_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  if (dbeta && ((uintptr_t)dbeta & 3u)) return fail(RACE_ERR_INVALID_ARG, "dbeta must be 4-byte aligned");
  if (dW && ((uintptr_t)dW & 3u)) return fail(RACE_ERR_INVALID_ARG, "dW must be 4-byte aligned");
  if (dW && !p.ks->dw_partial) return fail(RACE_ERR_UNSUPPORTED, "dW is not compiled for this (dtype, d, P, L)");
  const size_t dw_out = dW ? dw_out_floats(p) * sizeof(float) : 0;
  const size_t tbytes = (size_t)(p.BH * p.N * p.d) * elem_size(p.dtype);
  if (!p.causal) O = nullptr;   // the non-causal backward never reads O
  const void* ins[] = {Q, K, V, dO, O};
  void* outs[] = {dQ, dK, dV};
  for (void* o : outs) {
    for (const void* i : ins)
      if (overlaps(o, tbytes, i, tbytes)) return fail(RACE_ERR_INVALID_ARG, "an output overlaps an input");
    for (void* o2 : outs)
      if (o2 != o && overlaps(o, tbytes, o2, tbytes)) return fail(RACE_ERR_INVALID_ARG, "outputs overlap");
    if (overlaps(o, tbytes, dbeta, sizeof(float))) return fail(RACE_ERR_INVALID_ARG, "dbeta overlaps an output");
    if (overlaps(o, tbytes, dW, dw_out)) return fail(RACE_ERR_INVALID_ARG, "dW overlaps an output");
  }
  for (const void* i : ins) {
    if (overlaps(i, tbytes, dbeta, sizeof(float))) return fail(RACE_ERR_INVALID_ARG, "dbeta overlaps an input");
    if (overlaps(i, tbytes, dW, dw_out)) return fail(RACE_ERR_INVALID_ARG, "dW overlaps an input");
  }
  if (overlaps(dW, dw_out, dbeta, sizeof(float))) return fail(RACE_ERR_INVALID_ARG, "dW overlaps dbeta");
  if (overlaps(dW, dw_out, W, dw_out_floats(p) * sizeof(float))) return fail(RACE_ERR_INVALID_ARG, "dW overlaps W");
  const size_t need_state = state_bytes(p);
  if (state && state_bytes_in < need_state)
    return fail(RACE_ERR_WORKSPACE, "state too small: need " + std::to_string(need_state) + " bytes");
  const size_t need_ws = total_workspace_bytes(p, true, dW != nullptr, state == nullptr);
  if (!workspace || workspace_bytes_in < need_ws)
    return fail(RACE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need_ws) + " bytes" +
                                        (dW ? " (backward with dW)" : "") +
                                        (state ? "" : " (backward without a state)"));
  if (overlaps(dW, dw_out, workspace, need_ws)) return fail(RACE_ERR_INVALID_ARG, "dW overlaps the workspace");
  if (overlaps(dbeta, sizeof(float), workspace, need_ws))
    return fail(RACE_ERR_INVALID_ARG, "dbeta overlaps the workspace");
  if (state) {
    for (const void* o : outs)
      if (overlaps(state, need_state, o, tbytes)) return fail(RACE_ERR_INVALID_ARG, "state overlaps an output");
    if (overlaps(state, need_state, workspace, need_ws))
      return fail(RACE_ERR_INVALID_ARG, "state overlaps the workspace");
    if (overlaps(state, need_state, dbeta, sizeof(float))) return fail(RACE_ERR_INVALID_ARG, "state overlaps dbeta");
    if (overlaps(state, need_state, dW, dw_out)) return fail(RACE_ERR_INVALID_ARG, "state overlaps dW");
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (p.d == p.D) return bwd_run(p, Q, K, V, W, beta, O, dO, dQ, dK, dV, dbeta, dW, state, ws, s);
  // the caller's head dim is below the kernels': zero-padded copies of the
  // token tensors at the end of the workspace (Q, K, V, dO, O, dQ, dK, dV)
  char* r = ws + workspace_bytes(p, true, dW != nullptr, state == nullptr);
  const size_t tb = padded_tensor_bytes(p);
  void* kt[8];
  for (int i = 0; i < 8; ++i) kt[i] = r + i * tb;
  const void* src[] = {Q, K, V, dO, O};
  if ((st = copy_rows(p, src, kt, 5, true, s)) != RACE_OK) return st;
  st = bwd_run(p, kt[0], kt[1], kt[2], W, beta, O ? kt[4] : nullptr, kt[3], kt[5], kt[6], kt[7], dbeta, dW, state, ws,
               s);
  if (st != RACE_OK) return st;
  const void* grads[] = {kt[5], kt[6], kt[7]};
  void* outs_c[] = {dQ, dK, dV};
  return copy_rows(p, grads, outs_c, 3, false, s);
}

// ---- recurrent decode: the state is the bank [BH][LRP][d] + mass [BH][LRP]
race_status decode_plan(const race_shape* shape, int P, int L, Plan* p) {
  race_status st = make_plan(shape, P, L, 0, p, false);
  if (st != RACE_OK) return st;
  p->ks = nullptr;
  for (int D : kHeadDims) {
    if (D < p->d) continue;
    if ((p->ks = find_decode_set(p->dtype, D, p->PE, p->LRP))) {
      p->D = D;
      break;
    }
  }
  if (!p->ks) return fail(RACE_ERR_UNSUPPORTED, "no compiled kernel for this (dtype, d, P, L)");
  p->LRP = p->ks->LRP;
  return RACE_OK;
}

size_t race_attn_decode_state_bytes(const race_shape* shape, int P, int L) {
  Plan p;
  if (decode_plan(shape, P, L, &p) != RACE_OK) return 0;
  return bank_bytes(p);
}

size_t race_attn_decode_prefill_workspace_bytes(const race_shape* shape, int P, int L) {
  Plan p;
  if (decode_plan(shape, P, L, &p) != RACE_OK) return 0;
  return align256(part_bytes(p)) + pad_bytes(p, 2);
}

race_status race_attn_decode_prefill(const void* K, const void* V, const float* W, float beta, int P, int L,
                                     const race_shape* shape, void* state, size_t state_bytes_in, void* workspace,
                                     size_t workspace_bytes_in, race_stream_t stream) {
  g_last_error.clear();
  Plan p;
  race_status st = decode_plan(shape, P, L, &p);
  if (st != RACE_OK) return st;
  if (!K || !V || !W || !state) return fail(RACE_ERR_INVALID_ARG, "K, V, W and state must be non-NULL");
  if (!std::isfinite(beta)) return fail(RACE_ERR_INVALID_ARG, "beta must be finite");
  if (!aligned16(K) || !aligned16(V) || !aligned16(W) || !aligned16(state) || (workspace && !aligned16(workspace)))
    return fail(RACE_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  const size_t tbytes = (size_t)(p.BH * p.N * p.d) * elem_size(p.dtype);
  const size_t need_state = bank_bytes(p), need_ws = align256(part_bytes(p)) + pad_bytes(p, 2);
  if (state_bytes_in < need_state)
    return fail(RACE_ERR_WORKSPACE, "state too small: need " + std::to_string(need_state) + " bytes");
  if (!workspace || workspace_bytes_in < need_ws)
    return fail(RACE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need_ws) + " bytes");
  if (overlaps(state, need_state, K, tbytes) || overlaps(state, need_state, V, tbytes) ||
      overlaps(state, need_state, workspace, need_ws))
    return fail(RACE_ERR_INVALID_ARG, "state overlaps an input or the workspace");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(workspace);
  float* content = static_cast<float*>(state);
  float* mass = content + (size_t)p.BH * p.LRP * p.D;
  if (p.d != p.D) {
    // zero-padded copies of K and V after the partial banks
    char* r = static_cast<char*>(workspace) + align256(part_bytes(p));
    void* kt[2] = {r, r + padded_tensor_bytes(p)};
    const void* src[] = {K, V};
    if ((st = copy_rows(p, src, kt, 2, true, s)) != RACE_OK) return st;
    K = kt[0];
    V = kt[1];
  }
  race::NCArgs a{};
  a.X = K; a.Y = V; a.W = tables(p, W); a.beta = beta; a.L = p.L; a.P = p.P; a.N = p.N;
  a.part = part; a.chunk_tokens = p.chunk_tokens; a.nchunk = p.nchunk;
  {
    ProfScope ps(s, "race_bucket_reduce");
    p.ks->reduce(a, dim3(p.nchunk, (unsigned)p.BH), s);
  }
  if ((st = check_launch("race_bucket_reduce")) != RACE_OK) return st;
  {
    ProfScope ps(s, "race_bank_finalize");
    launch_finalize(part, p.nchunk, p, content, mass, s);
  }
  return check_launch("race_bank_finalize");
}

race_status race_attn_decode(const void* Q, const void* K, const void* V, const float* W, float beta, int P, int L,
                             void* O, const race_shape* shape, void* state, size_t state_bytes_in,
                             race_stream_t stream) {
  g_last_error.clear();
  Plan p;
  race_status st = decode_plan(shape, P, L, &p);
  if (st != RACE_OK) return st;
  if (!Q || !K || !V || !W || !O || !state) return fail(RACE_ERR_INVALID_ARG, "Q, K, V, W, O and state must be non-NULL");
  if (!std::isfinite(beta)) return fail(RACE_ERR_INVALID_ARG, "beta must be finite");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(W) || !aligned16(O) || !aligned16(state))
    return fail(RACE_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  const size_t tbytes = (size_t)(p.BH * p.N * p.d) * elem_size(p.dtype);
  const size_t need_state = bank_bytes(p);
  if (state_bytes_in < need_state)
    return fail(RACE_ERR_WORKSPACE, "state too small: need " + std::to_string(need_state) + " bytes");
  if (overlaps(O, tbytes, Q, tbytes) || overlaps(O, tbytes, K, tbytes) || overlaps(O, tbytes, V, tbytes))
    return fail(RACE_ERR_INVALID_ARG, "O overlaps an input");
  if (overlaps(state, need_state, O, tbytes) || overlaps(state, need_state, Q, tbytes) ||
      overlaps(state, need_state, K, tbytes) || overlaps(state, need_state, V, tbytes))
    return fail(RACE_ERR_INVALID_ARG, "state overlaps a token buffer");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  race::DArgs a{};
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.W = tables(p, W); a.beta = beta; a.L = p.L; a.P = p.P; a.N = p.N;
  a.dr = (int)p.d;
  a.content = static_cast<float*>(state);
  a.mass = a.content + (size_t)p.BH * p.LRP * p.D;
  {
    ProfScope ps(s, "race_decode");
    p.ks->decode(a, (unsigned)p.BH, s);
  }
  return check_launch("race_decode");
}

int race_bucket_stats_segments(const race_shape* shape, int P, int L, int causal, int64_t* seg_tokens) {
  Plan p;
  if (make_plan(shape, P, L, causal, &p, true) != RACE_OK) return 0;
  if (seg_tokens) *seg_tokens = p.causal ? p.seg_tokens : p.N;
  return p.causal ? p.nseg : 1;
}

race_status race_bucket_stats_debug(const race_shape* shape, int P, int L, int causal, const void* state,
                                    size_t state_bytes_in, const void* bwd_workspace, size_t bwd_workspace_bytes,
                                    float* content, float* mass, float* dcontent, float* dmass,
                                    race_stream_t stream) {
  g_last_error.clear();
  Plan p;
  race_status st = make_plan(shape, P, L, causal, &p, true);
  if (st != RACE_OK) return st;
  const bool fwd_out = content || mass, bwd_out = dcontent || dmass;
  if (!fwd_out && !bwd_out) return fail(RACE_ERR_INVALID_ARG, "no output requested");
  if (fwd_out && !state) return fail(RACE_ERR_INVALID_ARG, "content / mass need the forward's state");
  if (bwd_out && !bwd_workspace) return fail(RACE_ERR_INVALID_ARG, "dcontent / dmass need the backward's workspace");
  if (fwd_out && state_bytes_in < state_bytes(p))
    return fail(RACE_ERR_WORKSPACE, "state too small: need " + std::to_string(state_bytes(p)) + " bytes");
  if (bwd_out && bwd_workspace_bytes < workspace_bytes(p, true))
    return fail(RACE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(workspace_bytes(p, true)) +
                                        " bytes");
  for (const void* q : {(const void*)content, (const void*)mass, (const void*)dcontent, (const void*)dmass})
    if (q && ((uintptr_t)q & 3u)) return fail(RACE_ERR_INVALID_ARG, "outputs must be 4-byte aligned");
  const int64_t nbank = p.BH * (p.causal ? p.nseg : 1);
  const int R = 1 << P;
  const size_t per_c = (size_t)L * R * p.d * sizeof(float), per_m = (size_t)L * R * sizeof(float);
  const void* outs[] = {content, mass, dcontent, dmass};
  const size_t sizes[] = {nbank * per_c, nbank * per_m, nbank * per_c, nbank * per_m};
  for (int i = 0; i < 4; ++i) {
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], sizes[i], outs[j], sizes[j])) return fail(RACE_ERR_INVALID_ARG, "outputs overlap");
    if (overlaps(outs[i], sizes[i], state, state_bytes(p)) ||
        overlaps(outs[i], sizes[i], bwd_workspace, workspace_bytes(p, true)))
      return fail(RACE_ERR_INVALID_ARG, "an output overlaps the state or the workspace");
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t total = nbank * L * R * (p.d + 1);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  const int DP1 = (int)p.D + 1;
  const char* ws = static_cast<const char*>(bwd_workspace);
  const float gscale = 1.f / (float)(1 << (p.PE - P));
  if (fwd_out) {
    const float* b = static_cast<const float*>(state);
    if (p.causal) {   // segment banks [BH][nseg][LRP][d+1]: the bank before each segment
      hipLaunchKernelGGL(race::race_bank_export, dim3(blocks), dim3(256), 0, s, b, (int64_t)p.LRP * DP1, DP1,
                         b + p.D, (int64_t)p.LRP * DP1, DP1, nbank, L, P, p.PE, (int)p.d, 1.f, content, mass);
    } else {          // content [BH][LRP][d], mass [BH][LRP]
      hipLaunchKernelGGL(race::race_bank_export, dim3(blocks), dim3(256), 0, s, b, (int64_t)p.LRP * p.D,
                         (int)p.D, b + (size_t)p.BH * p.LRP * p.D, (int64_t)p.LRP, 1, nbank, L, P, p.PE,
                         (int)p.d, 1.f, content, mass);
    }
    if ((st = check_launch("race_bank_export")) != RACE_OK) return st;
  }
  if (bwd_out) {
    if (p.causal) {   // gradient banks after each segment [BH][nseg][LRP][d+1]
      const float* g = reinterpret_cast<const float*>(ws + causal_bwd_ws(p).gsuf);
      hipLaunchKernelGGL(race::race_bank_export, dim3(blocks), dim3(256), 0, s, g, (int64_t)p.LRP * DP1, DP1,
                         g + p.D, (int64_t)p.LRP * DP1, DP1, nbank, L, P, p.PE, (int)p.d, gscale, dcontent, dmass);
    } else {          // gradient bank dcontent [BH][LRP][d], dmass [BH][LRP]
      const float* g = reinterpret_cast<const float*>(ws + align256(nc_part_bytes(p)));
      hipLaunchKernelGGL(race::race_bank_export, dim3(blocks), dim3(256), 0, s, g, (int64_t)p.LRP * p.D,
                         (int)p.D, g + (size_t)p.BH * p.LRP * p.D, (int64_t)p.LRP, 1, nbank, L, P, p.PE,
                         (int)p.d, gscale, dcontent, dmass);
    }
    if ((st = check_launch("race_bank_export")) != RACE_OK) return st;
  }
  return RACE_OK;
}

race_status race_softbucket_debug(const void* X, const float* W, float beta, int P, int L, const race_shape* shape,
                                  float* phi_out, race_stream_t stream) {
  g_last_error.clear();
  Plan p;
  race_status st = make_plan(shape, P, L, 0, &p, true);
  if (st != RACE_OK) return st;
  if (P < 3) return fail(RACE_ERR_UNSUPPORTED, "the soft-assignment export needs P >= 3");
  if (!X || !W || !phi_out) return fail(RACE_ERR_INVALID_ARG, "X, W and phi_out must be non-NULL");
  if (!std::isfinite(beta)) return fail(RACE_ERR_INVALID_ARG, "beta must be finite");
  if (!aligned16(X) || !aligned16(W) || !aligned16(phi_out)) return fail(RACE_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
  int64_t blocks = (p.N + race::TT - 1) / race::TT;
  if (blocks > 4096) blocks = 4096;
  p.ks->softbucket_dbg(X, tables(p, W), beta, p.L, p.P, p.N, (int)p.d, phi_out, dim3((unsigned)blocks, (unsigned)p.BH),
                       reinterpret_cast<hipStream_t>(stream));
  return check_launch("race_softbucket_dbg");
}

const char* race_status_string(race_status status) {
  switch (status) {
    case RACE_OK: return "RACE_OK";
    case RACE_ERR_INVALID_ARG: return "RACE_ERR_INVALID_ARG";
    case RACE_ERR_UNSUPPORTED: return "RACE_ERR_UNSUPPORTED";
    case RACE_ERR_WORKSPACE: return "RACE_ERR_WORKSPACE";
    case RACE_ERR_HIP: return "RACE_ERR_HIP";
  }
  return "RACE_ERR_UNKNOWN";
}

const char* race_last_error(void) { return g_last_error.c_str(); }

race_status race_profile_enable(int on) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_on = on != 0;
  return RACE_OK;
}

void race_profile_reset(void) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (auto& r : g_prof_recs) {
    g_prof_pool.push_back(r.start);
    g_prof_pool.push_back(r.stop);
  }
  g_prof_recs.clear();
}

size_t race_profile_report(char* buf, size_t len) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  std::map<std::string, std::pair<int, double>> agg;
  for (auto& r : g_prof_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess) continue;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) continue;
    auto& a = agg[r.name];
    a.first += 1;
    a.second += ms;
  }
  std::string out;
  for (auto& kv : agg) {
    char line[256];
    std::snprintf(line, sizeof(line), "%s\t%d\t%.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    out += line;
  }
  if (buf && len) {
    std::size_t n = out.size() < len - 1 ? out.size() : len - 1;
    std::memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  return out.size() + 1;
}

}  // extern "C"
