// Causal RACE attention for gfx950: prefix bucket sums (slides frame
// "Causality is a prefix update of the same statistics", paper Algorithm 2;
// reading notes section 2.6).  The key at position t is added before the
// query at t reads, so token t sees keys j <= t.
//
// The sequence of every (batch, head) is cut into segments; the bank at each
// segment start comes from a segment-sum walk plus an exclusive scan over
// segments.  Contractions of the bank over buckets (O, den, h, dV) run in the
// cooperative readout-layout walks of race_walk.hpp.  This file holds the
// walks that contract the bank over value columns:
//   race_causal_transposed  one wave per window of whole tables (bucket
//                           rows): dPhi_Q on a forward walk, dPhi_K on a
//                           reverse walk, then softmax, tanh and projection
//                           backward of those tables.
// Backward (exact gradient of the causal forward map, W and beta fixed):
//   g_t = dO_t / Den_t,  h_t = -(dO_t . O_t) / Den_t
//   dPhi_Q,t = sum_{j<=t} phi_K,j (V_j . g_t + h_t)          (forward walk)
//   dPhi_K,j = sum_{t>=j} phi_Q,t (g_t . V_j + h_t)          (reverse walk)
// and dQ, dK = dPre . W.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/race_attn.h"
#include "race_noncausal.hpp"
#include "race_registry.hpp"

namespace race {

constexpr int CC = 32;   // tokens per causal chunk

struct CArgs {
  const void* A_src;      // rows whose features take the output (query) role
  const void* B_src;      // rows whose features take the state (key) role
  const void* X_src;      // value rows of the state role (V; or dO, divided by Den)
  const void* U_src;      // value rows of the output role (transposed kernel: dO or V)
  float* dpre_out;        // transposed: [BH][N][NHP] dPre of the output role
  const float* W;
  const float* seg_state; // [BH][nseg][LRP][d+1]: bank before (forward walk) / after (reverse walk) the segment
  const float* den;       // [BH][N]
  const float* hvec;      // [BH][N]
  float beta;
  int L, P;
  int64_t N;
  int64_t seg_tokens;
  int nseg;
  int64_t units;
};

// Segments: about 1024 (segment, batch x head) units over the whole problem,
// 64-token multiples.
inline void causal_segmentation(int64_t N, int64_t BH, int* nseg, int64_t* seg_tokens) {
  int64_t want = (1024 + BH - 1) / BH;
  const int64_t tiles = (N + 63) / 64;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t per = (tiles + want - 1) / want;
  *seg_tokens = per * 64;
  *nseg = (int)((N + *seg_tokens - 1) / *seg_tokens);
}

// ------------------------------------------------------------------ race_causal_transposed
// Unit = (segment, bh, window TG of whole tables).  Bank rows of the window
// live in acc[a][ct] as C[c][lr] tiles (lane = bucket row, registers over
// value columns c; tile CT holds the mass / h column at c = d).
// Forward walk (dPhi_Q): output role Q, state role K, X = [V | 1], U = [g | h].
// Reverse walk (dPhi_K):  output role K, state role Q, X = [g | h], U = [V | 1].
template <typename T, class G, bool REV, int TG>
__device__ __forceinline__ void transposed_body(const CArgs& a, int64_t seg, int64_t bh,
                                                const typename Eng<T>::frag* __restrict__ Wf, T* __restrict__ PhiT,
                                                T* __restrict__ Xh, T* __restrict__ Xl) {
  using E = Eng<T>;
  using frag = typename E::frag;
  constexpr int NS = E::NSPLIT;
  constexpr int URP = G::R > 32 ? G::R : 32;
  constexpr int ATU = URP / 32;
  constexpr int R0 = TG * URP;
  constexpr int TTP = CC + 8;
  constexpr int XSP = G::D + 32 + 8;
  constexpr int NC = G::CT + 1;          // column tiles incl. the mass / h tile
  constexpr bool XEXACT = !REV;          // X = [V | 1] is exact in T; [g | h] is not
  constexpr bool UEXACT = REV;           // U = [V | 1] exact; [g | h] not
  constexpr bool USE_XL = !XEXACT && NS == 2;
  const int lane = lane_id(), n = lane & 31, h = lane >> 5;
  const int64_t s0 = seg * a.seg_tokens, s1 = min(a.N, s0 + a.seg_tokens);
  const size_t rb = (size_t)bh * a.N;
  const T* Ar = static_cast<const T*>(a.A_src) + rb * G::D;
  const T* Br = static_cast<const T*>(a.B_src) + rb * G::D;
  const T* Xr = static_cast<const T*>(a.X_src) + rb * G::D;
  const T* Ur = static_cast<const T*>(a.U_src) + rb * G::D;
  const float* den = a.den + rb;
  const float* hv = a.hvec + rb;

  f32x16 acc[ATU][NC];
  {
    const float* ss = a.seg_state + ((size_t)bh * a.nseg + seg) * G::LRP * (G::D + 1);
#pragma unroll
    for (int at = 0; at < ATU; ++at)
#pragma unroll
      for (int ct = 0; ct < NC; ++ct)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int c = 32 * ct + 8 * (v >> 2) + 4 * h + (v & 3);
          const int lr = R0 + 32 * at + n;
          acc[at][ct][v] = (c <= G::D) ? ss[(size_t)lr * (G::D + 1) + c] : 0.f;
        }
  }
  // the mass-tile columns past c = d stay zero in the X tiles
  for (int r = 0; r < CC; ++r) {
    if (lane < 32) {
      Xh[r * XSP + G::D + lane] = (T)0.f;
      if (USE_XL) Xl[r * XSP + G::D + lane] = (T)0.f;
    }
  }
  const float beta2 = 2.f * a.beta;
  const int64_t nch = (s1 - s0 + CC - 1) / CC;
  for (int64_t k = 0; k < nch; ++k) {
    const int64_t t0 = s0 + (REV ? (nch - 1 - k) : k) * CC;
    const int64_t tok = t0 + n;
    const bool valid = tok < s1;
    // output-role features of the window (float32, for the softmax backward)
    float uA[G::NHP], phA[URP / 2];
    {
      frag xf[G::KD];
      float pre[G::NHP];
      load_row_frags<T, G>(valid ? Ar + tok * G::D : nullptr, xf);
      project<T, G>(Wf, xf, pre);
      soft_assign_rows<G, R0, URP>(pre, beta2, a.L, uA, phA);
    }
    // state-role features of the window, rounded, transposed into LDS
    {
      frag xf[G::KD];
      float pre[G::NHP], uB[G::NHP], phB[URP / 2];
      load_row_frags<T, G>(valid ? Br + tok * G::D : nullptr, xf);
      project<T, G>(Wf, xf, pre);
      soft_assign_rows<G, R0, URP>(pre, beta2, a.L, uB, phB);
#pragma unroll
      for (int at = 0; at < ATU; ++at)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = 32 * at + 8 * (v >> 2) + 4 * h + (v & 3);
          PhiT[lr * TTP + n] = valid ? (T)phB[16 * at + v] : (T)0.f;
        }
    }
    // output-role values U in TLAYOUT over columns (tile CT: c = d only)
    float ut[NC * 16];
    {
      float tmp[G::D / 2];
      if (valid) load_tl_row<T, G::D>(Ur + tok * G::D, tmp);
      else {
#pragma unroll
        for (int i = 0; i < G::D / 2; ++i) tmp[i] = 0.f;
      }
      const float scale = (!REV && valid) ? 1.f / den[tok] : 1.f;
#pragma unroll
      for (int i = 0; i < G::D / 2; ++i) ut[i] = tmp[i] * scale;
#pragma unroll
      for (int i = 0; i < 16; ++i) ut[G::D / 2 + i] = 0.f;
      const float extra = REV ? 1.f : (valid ? hv[tok] : 0.f);
      if (h == 0) ut[G::D / 2] = valid ? extra : 0.f;
    }
    // state-role values X: rows t0..t0+31, columns 0..d (c = d: 1 or h)
    {
      constexpr int EPC = 16 / (int)sizeof(T);
      constexpr int CPR = G::D / EPC;
#pragma unroll
      for (int it = 0; it < 32 * CPR / 64; ++it) {
        const int flat = it * 64 + lane;
        const int row = flat / CPR, ch = flat % CPR;
        const int64_t tr = t0 + row;
        float f[EPC];
#pragma unroll
        for (int kk = 0; kk < EPC; ++kk) f[kk] = 0.f;
        if (tr < s1) {
          const uint4 val = *reinterpret_cast<const uint4*>(Xr + tr * G::D + ch * EPC);
          const T* e = reinterpret_cast<const T*>(&val);
          const float sc = REV ? 1.f / den[tr] : 1.f;
#pragma unroll
          for (int kk = 0; kk < EPC; ++kk) f[kk] = (float)e[kk] * sc;
        }
#pragma unroll
        for (int kk = 0; kk < EPC; ++kk) {
          const T hi = (T)f[kk];
          Xh[row * XSP + ch * EPC + kk] = hi;
          if (USE_XL) Xl[row * XSP + ch * EPC + kk] = (T)(f[kk] - (float)hi);
        }
      }
      if (h == 0) {
        const float m = (!valid) ? 0.f : (REV ? hv[tok] : 1.f);
        const T hi = (T)m;
        Xh[n * XSP + G::D] = hi;
        if (USE_XL) Xl[n * XSP + G::D] = (T)(m - (float)hi);
      }
    }
    wave_lds_sync();

    // dPhi of the output role, rows of the window: inter part from the bank
    f32x16 dp[ATU];
#pragma unroll
    for (int at = 0; at < ATU; ++at) dp[at] = zero16();
#pragma unroll
    for (int q = 0; q < 2 * NC; ++q) {
      frag uh, ul;
      {
        float u8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) u8[i] = ut[8 * q + i];
        E::split(u8, uh, ul);
      }
#pragma unroll
      for (int at = 0; at < ATU; ++at) {
        float v8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = acc[at][q >> 1][8 * (q & 1) + i];
        frag ah, al;
        E::split(v8, ah, al);
        E::mma(ah, uh, dp[at]);
        if (NS == 2) {
          if (!UEXACT) E::mma(ah, ul, dp[at]);
          E::mma(al, uh, dp[at]);
        }
      }
    }
    // intra part: m^T[tok_b][tok_a] = X_b . U_a (masked), then Phi_B^T m^T
    {
      f32x16 mf = zero16();
#pragma unroll
      for (int q = 0; q < 2 * NC; ++q) {
        frag uh, ul;
        {
          float u8[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) u8[i] = ut[8 * q + i];
          E::split(u8, uh, ul);
        }
        frag xh, xl;
#pragma unroll
        for (int i = 0; i < 8; ++i) xh[i] = Xh[n * XSP + kmap(q, h, i)];
        E::mma(xh, uh, mf);
        if (NS == 2) {
          if (!UEXACT) E::mma(xh, ul, mf);
          if (USE_XL) {
#pragma unroll
            for (int i = 0; i < 8; ++i) xl[i] = Xl[n * XSP + kmap(q, h, i)];
            E::mma(xl, uh, mf);
          }
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tb = 8 * (v >> 2) + 4 * h + (v & 3);
        const bool keep = REV ? (tb >= n) : (tb <= n);
        mf[v] = keep ? mf[v] : 0.f;
      }
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        float m8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) m8[i] = mf[8 * q2 + i];
        frag mh, ml;
        E::split(m8, mh, ml);
#pragma unroll
        for (int at = 0; at < ATU; ++at) {
          frag pf;
#pragma unroll
          for (int i = 0; i < 8; ++i) pf[i] = PhiT[(32 * at + n) * TTP + kmap(q2, h, i)];
          E::mma(pf, mh, dp[at]);
          if (NS == 2) E::mma(pf, ml, dp[at]);
        }
      }
    }
    // softmax, tanh backward of the window's tables -> dPre
    {
      float dphi[URP / 2];
#pragma unroll
      for (int at = 0; at < ATU; ++at)
#pragma unroll
        for (int v = 0; v < 16; ++v) dphi[16 * at + v] = dp[at][v];
      float dpre[G::NHP];
#pragma unroll
      for (int i = 0; i < G::NHP; ++i) dpre[i] = 0.f;
      assign_backward_rows<G, R0, URP>(phA, dphi, uA, a.beta, dpre);
      constexpr int L0 = R0 / G::R;
      constexpr int L1 = cdiv(R0 + URP, G::R) < G::LMAX ? cdiv(R0 + URP, G::R) : G::LMAX;
      if (valid && h == 0) {
        float* dst = a.dpre_out + (rb + tok) * G::NHP;
#pragma unroll
        for (int hp = L0 * G::PE; hp < L1 * G::PE; ++hp) dst[hp] = dpre[hp];
      }
    }
    // bank update: C[c][lr] += X^T[c][tok] Phi_B[tok][lr]
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      frag pfs[ATU];
#pragma unroll
      for (int at = 0; at < ATU; ++at)
        pfs[at] = *reinterpret_cast<const frag*>(PhiT + (32 * at + n) * TTP + 16 * s + 8 * h);
#pragma unroll
      for (int ct = 0; ct < NC; ++ct) {
        frag xh, xl;
#pragma unroll
        for (int i = 0; i < 8; ++i) xh[i] = Xh[(16 * s + 8 * h + i) * XSP + 32 * ct + n];
        if (USE_XL) {
#pragma unroll
          for (int i = 0; i < 8; ++i) xl[i] = Xl[(16 * s + 8 * h + i) * XSP + 32 * ct + n];
        }
#pragma unroll
        for (int at = 0; at < ATU; ++at) {
          E::mma(xh, pfs[at], acc[at][ct]);
          if (USE_XL) E::mma(xl, pfs[at], acc[at][ct]);
        }
      }
    }
    wave_lds_sync();
  }
}

template <typename T, class G, bool REV, int TG>
__device__ __forceinline__ void transposed_dispatch(int tg, const CArgs& a, int64_t seg, int64_t bh,
                                                    const typename Eng<T>::frag* Wf, T* PhiT, T* Xh, T* Xl) {
  constexpr int URP = G::R > 32 ? G::R : 32;
  if (tg == TG) {
    transposed_body<T, G, REV, TG>(a, seg, bh, Wf, PhiT, Xh, Xl);
  } else if constexpr ((TG + 1) * URP < G::LRP) {
    transposed_dispatch<T, G, REV, TG + 1>(tg, a, seg, bh, Wf, PhiT, Xh, Xl);
  }
}

template <typename T, class G, bool REV>
__global__ __launch_bounds__(256) void race_causal_transposed(CArgs a) {
  using E = Eng<T>;
  using frag = typename E::frag;
  constexpr int URP = G::R > 32 ? G::R : 32;
  constexpr int NTG = G::LRP / URP;
  constexpr int TTP = CC + 8;
  constexpr int XSP = G::D + 32 + 8;
  constexpr bool USE_XL = REV && E::NSPLIT == 2;   // X = [g | h] needs hi + lo parts
  __shared__ frag Wf[G::NPT * G::KD * 64];
  __shared__ T PhiT_all[4][URP * TTP];
  __shared__ T Xh_all[4][CC * XSP];
  __shared__ T Xl_all[USE_XL ? 4 : 1][CC * XSP];
  build_proj_frags<T, G>(a.W, a.L, a.P, Wf);
  __syncthreads();
  const int w = threadIdx.x >> 6;
  const int64_t unit = (int64_t)blockIdx.x * 4 + w;
  if (unit >= a.units) return;
  const int tg = (int)(unit % NTG);
  const int64_t seg = (unit / NTG) % a.nseg;
  const int64_t bh = unit / NTG / a.nseg;
  transposed_dispatch<T, G, REV, 0>(tg, a, seg, bh, Wf, PhiT_all[w], Xh_all[w], Xl_all[USE_XL ? w : 0]);
}

// ------------------------------------------------------------------ dX = dPre . W
template <typename T, class G>
__global__ __launch_bounds__(256) void race_dx(const float* __restrict__ dpre, const float* __restrict__ W, int L,
                                               int P, int64_t N, int64_t BH, void* __restrict__ outv) {
  using E = Eng<T>;
  using frag = typename E::frag;
  __shared__ frag WTf[G::CT * G::NQS * 64];
  build_wt_frags<T, G>(W, L, P, WTf);
  __syncthreads();
  const int lane = lane_id(), n = lane & 31, w = threadIdx.x >> 6;
  const int64_t total = BH * N;
  T* out = static_cast<T*>(outv);
  for (int64_t base = (int64_t)blockIdx.x * TT + 32 * w; base < total; base += (int64_t)gridDim.x * TT) {
    const int64_t tok = base + n;
    const bool valid = tok < total;
    float dp[G::NHP];
#pragma unroll
    for (int i = 0; i < G::NHP; ++i) dp[i] = valid ? dpre[tok * G::NHP + i] : 0.f;
    float dx[G::D / 2];
    dx_mma<T, G>(WTf, dp, dx);
    if (valid) store_tl_row<T, G::D>(out + tok * G::D, dx);
  }
}

// ------------------------------------------------------------------ small kernels
// Exclusive scan over segments (forward: banks before each segment; reverse:
// banks after it), one thread per (bh, bank element).
static __global__ void race_seg_scan(const float* __restrict__ part, float* __restrict__ out, int nseg, int per, int BH,
                              int reverse) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)BH * per) return;
  const int64_t bh = idx / per, rem = idx % per;
  float run = 0.f;
  for (int k = 0; k < nseg; ++k) {
    const int s = reverse ? nseg - 1 - k : k;
    const size_t o = ((size_t)bh * nseg + s) * per + rem;
    const float v = part[o];
    out[o] = run;
    run += v;
  }
}

}  // namespace race
