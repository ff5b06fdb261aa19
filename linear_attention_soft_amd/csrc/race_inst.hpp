// Launchers of one kernel instance; included by the per-dtype instance files.
#pragma once
#include "race_causal.hpp"
#include "race_noncausal.hpp"
#include "race_registry.hpp"
#include "race_walk.hpp"
#include "race_decode.hpp"
#include "race_dw.hpp"

namespace race {

// race_dw_partial takes the non-causal chunking's workgroup count, which never
// exceeds the number of 128-token tiles: each of its workgroups gets a tile.
static_assert(DW_TT == TT, "dW tiles are the non-causal tiles");

// Soft assignments of token rows written out as float32 [BH][N][L][R]
// (a test export of the fused front end every kernel uses).  Token rows have
// dr <= D elements (a multiple of 8); the kernel's columns past dr are zero.
template <typename T, class G>
__global__ __launch_bounds__(256) void race_softbucket_dbg(const void* Xv, Tables W, float beta,
                                                           int L, int P, int64_t N, int dr, float* out) {
  using E = Eng<T>;
  using frag = typename E::frag;
  __shared__ frag Wf[G::NPT * G::KD * 64];
  const int bh = blockIdx.y;
  build_proj_frags<T, G>(W.at(bh), W.ld, L, P, Wf);
  __syncthreads();
  const int lane = lane_id(), n = lane & 31, h = lane >> 5, w = threadIdx.x >> 6;
  const T* X = static_cast<const T*>(Xv) + (size_t)bh * N * dr;
  const int LR = L << G::PE;
  for (int64_t base = (int64_t)blockIdx.x * TT + 32 * w; base < N; base += (int64_t)gridDim.x * TT) {
    const int64_t tok = base + n;
    const bool valid = tok < N;
    frag xf[G::KD];
#pragma unroll
    for (int q = 0; q < G::KD; ++q) {
      const int c0 = 16 * q + 8 * h;   // 8 consecutive columns, all inside dr or all past it
      xf[q] = (valid && c0 < dr) ? *reinterpret_cast<const frag*>(X + tok * dr + c0) : E::zero();
    }
    float pre[G::NHP], ev[G::NHP], phi[G::LRP / 2];
    project<T, G>(Wf, xf, pre);
    soft_assign<G>(pre, 2.f * beta, L, ev, phi);
    if (valid) {
#pragma unroll
      for (int at = 0; at < G::AT; ++at)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = 32 * at + 8 * (v >> 2) + 4 * h + (v & 3);
          if (lr < LR) out[((size_t)bh * N + tok) * LR + lr] = phi[16 * at + v];
        }
    }
  }
}

template <typename T, int D, int PE, int LRP>
struct Inst {
  using G = Geo<T, D, PE, LRP>;
  static unsigned blocks4(int64_t units) { return (unsigned)((units + 3) / 4); }
  static void reduce(const NCArgs& a, dim3 g, hipStream_t s) {
    hipLaunchKernelGGL((race_bucket_reduce<T, G>), g, dim3(256), 0, s, a);
  }
  static void readout(const NCArgs& a, dim3 g, hipStream_t s) {
    hipLaunchKernelGGL((race_readout_norm<T, G>), g, dim3(256), 0, s, a);
  }
  static void bwd_q(const NCArgs& a, dim3 g, hipStream_t s) {
    hipLaunchKernelGGL((race_bwd_q<T, G>), g, dim3(256), 0, s, a);
  }
  static void bwd_kv(const NCArgs& a, dim3 g, hipStream_t s) {
    hipLaunchKernelGGL((race_bwd_kv<T, G>), g, dim3(256), 0, s, a);
  }
  static void dbg(const void* X, const Tables& W, float beta, int L, int P, int64_t N, int dr, float* out,
                  dim3 g, hipStream_t s) {
    hipLaunchKernelGGL((race_softbucket_dbg<T, G>), g, dim3(256), 0, s, X, W, beta, L, P, N, dr, out);
  }
  template <int MODE>
  static void walk(const WArgs& a, dim3 g, hipStream_t s) {
    hipLaunchKernelGGL((race_walk_rw<T, G, MODE>), g, dim3(RWCfg<T, G, MODE>::NT), 0, s, a);
  }
  template <bool REV, bool STATIC = false>
  static void tw(const TWArgs& a, dim3 g, hipStream_t s) {
    hipLaunchKernelGGL((race_walk_tw<T, G, REV, STATIC>), g, dim3(TWCfg<T, G, REV, STATIC>::NT), 0, s, a);
  }
  static void h_from_o(const void* dO, const void* O, const float* den, float* h, int64_t total, hipStream_t s) {
    constexpr int LPT = D / (16 / (int)sizeof(T));
    const int64_t threads = total * LPT;
    hipLaunchKernelGGL((race_h_from_o<T, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       static_cast<const T*>(dO), static_cast<const T*>(O), den, h, total);
  }
  static void decode(const DArgs& a, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((race_decode<T, G>), dim3(grid), dim3(DecCfg<G>::NT), 0, s, a);
  }
  static void dw_partial(const DWArgs& a, dim3 g, hipStream_t s) {
    hipLaunchKernelGGL((race_dw_partial<T, G>), g, dim3(256), 0, s, a);
  }
  // NC: compile the non-causal kernels; CAUSAL: the causal ones; NCST: the
  // non-causal layer as static-bank walks (with the segment-sum walks)
  template <bool NC, bool CAUSAL, bool NCST = false>
  static KernelSet set(int dtype) {
    KernelSet k{};
    k.dtype = dtype; k.D = D; k.PE = PE; k.LRP = LRP; k.NHP = G::NHP;
    k.reduce = reduce;
    k.softbucket_dbg = dbg;
    k.decode = decode;
    // the table-gradient partials read dPre rows as float4: NHP a multiple of 4
    if constexpr (G::NHP % 4 == 0) k.dw_partial = dw_partial;
    if constexpr (NC) { k.readout = readout; k.bwd_q = bwd_q; k.bwd_kv = bwd_kv; }
    if constexpr (CAUSAL) {
      k.tw_dq = tw<false>; k.tw_dk = tw<true>; k.h_from_o = h_from_o;
      k.tw_pre = TWCfg<T, G, false, false>::PRE ? 1 : 0;
      k.w_segsum = walk<W_SEGSUM>; k.w_gsum = walk<W_GSUM>; k.w_fwd = walk<W_FWD>; k.w_h = walk<W_H>;
      k.w_dv = walk<W_DV>;
    }
    if constexpr (NCST) {
      k.w_segsum = walk<W_SEGSUM>; k.w_gsum = walk<W_GSUM>;
      k.w_fwd_st = walk<W_FWD_ST>; k.w_h_st = walk<W_H_ST>; k.w_dv_st = walk<W_DV_ST>;
      k.tw_dq_st = tw<false, true>; k.tw_dk_st = tw<true, true>;
    }
    return k;
  }
};

}  // namespace race
