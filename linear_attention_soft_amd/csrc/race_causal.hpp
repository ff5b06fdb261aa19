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
//   race_walk_tw  one wave per window of 32 bucket rows (whole tables, or a
//                 part of a table of 64 to 256 corners), the workgroup walking
//                 one (segment, batch x head): dPhi_Q on a forward walk,
//                 dPhi_K on a reverse walk, then softmax, tanh and projection
//                 backward of those tables and dX = dPre . W.
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
#include "race_walk.hpp"

namespace race {

// Segments, in 64-token multiples: about 256 (segment, batch x head) units
// over the whole problem, one per CU (a walk workgroup fills a CU), when each
// segment still gets at least 64 tiles; otherwise about 512.  Measured in one
// process on one set of buffers: the 1M-token, 4-head step 13.25 -> 13.09 ms
// with 256 units against 512 (768: 13.29); the 64 x 1K-token step keeps 512
// units of 128 tokens (0.221 ms; 256 units: 0.260; 1024 units: 0.259).
inline void causal_segmentation(int64_t N, int64_t BH, int* nseg, int64_t* seg_tokens) {
  const int64_t tiles = (N + 63) / 64;
  int64_t want = (256 + BH - 1) / BH;
  if (tiles / want < 64) want = (512 + BH - 1) / BH;
  if (want > tiles) want = tiles;
  if (want < 1) want = 1;
  const int64_t per = (tiles + want - 1) / want;
  *seg_tokens = per * 64;
  *nseg = (int)((N + *seg_tokens - 1) / *seg_tokens);
}

struct TWArgs {
  const void* A_src;      // output-role rows (forward walk: Q; reverse walk: K)
  const void* B_src;      // state-role rows (forward: K; reverse: Q)
  const void* X_src;      // state-role values: forward V; reverse dO (divided by den: g)
  const void* U_src;      // output-role values: forward dO; reverse V
  void* dX;               // dQ (forward) or dK (reverse)
  const float* bank_in;   // [BH][nseg][LRP][d+1]: bank before (forward) / after (reverse) the segment;
                          // static walks: content [BH][LRP][d]
  const float* mass_in;   // static walks: mass [BH][LRP]
  const float* den;       // [BH][N]
  const float* hvec;      // [BH][N]
  Tables W;
  float* dbeta_part;      // when set: [BH][nseg][waves] shares of dL/dbeta
  float* dpre_out;        // when set: dL/dPre of every token, float32 [BH][N][NHP]
  // causal walks: stored projections W x of the output and state roles
  // (float32 [BH][N][NHP], slot l PE + t), made once by the readout walks
  const float* preA_in;
  const float* preB_in;
  float beta;
  int L, P;
  int64_t N;
  int64_t seg_tokens;
  int nseg;
};

// One wave per window of 32 bucket rows: whole tables when 2^PE <= 32, else
// a 32-corner part of a table (SPL = 2^PE / 32 = 2, 4 or 8 waves per table,
// which exchange their softmax-backward sums once per chunk).  The workgroup
// walks one (segment, batch x head).
template <typename T, class G, bool REV, bool STATIC = false>
struct TWCfg {
  // STATIC: the non-causal layer for wide banks: every token of the
  // (batch, head) reads one fixed bank (segment index ignored); no state-role
  // rows, no intra-chunk term, no bank update
  static constexpr bool ST = STATIC;
  static constexpr int URP = 32;
  static constexpr int SPL = G::R > 32 ? G::R / 32 : 1;   // waves per table
  static_assert(G::PE <= 8 && SPL <= G::LRP / URP, "a table spans at most the workgroup's waves");
  static constexpr int NM = G::LRP / URP;             // waves
  static constexpr int ATU = URP / 32;                // 32-row tiles per wave
  static constexpr int NT = 64 * NM;
  static constexpr bool XSPLIT = REV && !STATIC && Eng<T>::NSPLIT == 2;   // X = dO / den is not exact in T
  // causal walks with split tables read both roles' stored projections
  // instead of staging the Q and K rows and projecting them (whole-table
  // waves would hold more slots in registers than they save; static walks
  // project)
  static constexpr bool PRE = !STATIC && SPL > 1;
  static constexpr int NXS = XSPLIT ? 2 : 1;
  // staged row (elements): with bf16 at d = 128, rows 76 dwords apart (12
  // mod 64 banks) keep both the 16-byte row reads and the transposing loads
  // of X free of bank conflicts.  d = 64 rows are 36 dwords apart,
  // conflict-free for both.
  static constexpr int FS = G::D + ((std::is_same<T, bf16>::value && G::D == 128) ? 24 : 16 / (int)sizeof(T));
  // Phi_B^T row (elements): an 88-byte stride keeps both its 2-byte transposed
  // writes (rows 4 apart fall 96 bytes apart) and its 8-byte operand reads (32
  // consecutive rows start on distinct 8-byte bank pairs) free of bank conflicts
  static constexpr int TSP = WC + 12;
  // bf16: the state-role features of the chunk are kept token-major per
  // wave (rows of the wave's URP bucket rows, RS elements apart) and read
  // transposed by transposing LDS loads (intra and bank-update operands,
  // bucket masses).  Rows 24 dwords apart: the four rows that one 16-lane
  // group of such a load reads fall on disjoint banks.  float32 keeps the
  // transposed copy (TSP-element rows per bucket row).
  static constexpr bool TRB = std::is_same<T, bf16>::value;
  static constexpr int RS = URP + 4;   // 18 dwords: the 8-byte row writes of the 32 tokens are conflict-free too
  // dPre row per token (floats): an odd number of 16-byte groups, so that 16
  // lanes' 16-byte accesses of 16 tokens fall on distinct banks
  static constexpr int DPS = 4 * ((cdiv(G::NHP, 4) | 1));
  // bf16: the waves that form dPre write the B operands of dX = dPre . W
  // directly, as one bf16 row per token whose entry e is the hi part of
  // dPre[e % NHP] (e < NHP or e >= 2 NHP) or its lo part (NHP <= e < 2 NHP),
  // matching the W^T entries (W hi, W hi, W lo); each K16 step of the dX MFMA
  // is then one 16-byte read.  Rows 4 (2 NQS + 1) dwords apart: the 16-byte
  // reads of 16 lanes fall on distinct banks.  Used where the stages still fit
  // the 160 KB of LDS with these rows (TWLds::DXB); otherwise float32 dPre
  // rows are kept and every dX wave builds the operands.
  static constexpr int DBS = 16 * G::NQS + 8;
  // Shared intra-chunk scores (TWLds::SHSC, with at least four waves and where
  // the LDS still fits): mf[b][a] (b: state-role token, a: output-role
  // token) is computed once per chunk as four 16 x 16 sub-tiles by four waves
  // and read by every wave as the B operand of its intra term, instead of
  // every wave forming the whole 32 x 32 tile.  One row per output token a
  // with entry b at the kmap frag position of b (bits 2 and 3 of b
  // exchanged); bf16 keeps hi and lo parts.  Rows 4 x odd dwords apart.
  static constexpr int MS = std::is_same<T, bf16>::value ? 40 : 36;
  static constexpr int NCTW = cdiv(G::CT, NM);        // dX column tiles per wave
  static constexpr int EPC = 16 / (int)sizeof(T);
  static constexpr int CPR = G::D / EPC;              // 16-byte chunks per value row
  static constexpr int NPS = cdiv(WC * CPR, NT);      // staged chunks per thread
  // The float32 bank enters the contraction over value columns as bf16
  // hi + lo parts (the softmax backward that follows subtracts nearly equal
  // terms).
  static constexpr bool BANK_LO = false;
  static_assert(G::LRP % URP == 0, "windows of 32 rows");
};

template <typename T, class G, bool REV, bool STATIC, bool DXB_, bool SHSC_>
struct TWLdsT {
  using C = TWCfg<T, G, REV, STATIC>;
  static constexpr bool DXB = DXB_, SHSC = SHSC_;
  // one buffer of dPre rows when a workgroup barrier separates the previous
  // chunk's dX reads (at the top of a chunk) from this chunk's dPre writes
  // (the shared-score barrier or the split-table exchange), two otherwise
  static constexpr int NDB = (SHSC || C::SPL > 1) ? 1 : 2;
  // one buffer of output-role, state-role and U rows when a workgroup barrier
  // (shared scores, split-table exchange) follows their last reads in a
  // chunk, so the next chunk's rows, staged at its end, cannot overwrite rows
  // another wave still reads; two otherwise.  X rows, read by the bank
  // update after those barriers, keep two.
  static constexpr int NSB = (SHSC || C::SPL > 1) ? 1 : 2;
  static constexpr int SROWS = STATIC ? 8 : WC * C::FS;   // state-role stages (none when static)
  // projection operands: shared 8- or 16-slot tiles, or one tile per table (SPL = 2)
  typename Eng<T>::frag Wf[C::PRE ? 1 : (C::SPL > 1 ? G::LMAX : G::NPT) * G::KD * 64];
  alignas(16) T PhiBT[C::NM][STATIC ? 8 : (C::TRB ? WC * C::RS : C::URP * C::TSP)];   // wave-private Phi_B
  alignas(16) float Mw[C::NM][C::URP];           // wave-private mass (forward) / h-weighted mass (reverse)
  alignas(16) T AR[NSB][C::PRE ? 8 : WC * C::FS];   // output-role rows (projection operands)
  alignas(16) T BR[NSB][C::PRE ? 8 : SROWS];        // state-role rows
  alignas(16) T UF[NSB][WC * C::FS];             // U rows, kmap frag order
  alignas(16) T XF[2][C::NXS][SROWS];            // X rows, kmap frag order (hi, lo)
  alignas(16) float DP[NDB][DXB ? 4 : WC * C::DPS];    // dPre of every table (float32 rows)
  alignas(16) T DB[NDB][DXB ? WC * C::DBS : 8];        // dX B-operand rows (bf16 I/O)
  alignas(16) T MFT[SHSC ? Eng<T>::NSPLIT : 1][SHSC ? WC * C::MS : 8];   // shared intra-chunk scores
  alignas(16) float TK[2][3][WC];                // per token: xe (X extra), ue (U extra), 1/den
  alignas(16) T XEB[2][2][C::TRB ? WC : 4];      // bf16: xe as hi + lo (mass sums on v_dot2)
  alignas(16) float XS[C::SPL > 1 ? C::NM : 1][G::PE + 1][WC];   // split-table softmax-backward sums
};

// Stage layout: shared scores first, then bf16 dX rows, as far as 160 KB allow.
constexpr size_t kLdsBytes = 160 * 1024;
template <typename T, class G, bool REV, bool STATIC>
struct TWPick {
  static constexpr bool BF = std::is_same<T, bf16>::value;
  static constexpr bool FIT_TT = sizeof(TWLdsT<T, G, REV, STATIC, true, true>) <= kLdsBytes;
  static constexpr bool FIT_FT = sizeof(TWLdsT<T, G, REV, STATIC, false, true>) <= kLdsBytes;
  static constexpr bool FIT_TF = sizeof(TWLdsT<T, G, REV, STATIC, true, false>) <= kLdsBytes;
  static constexpr bool SH = !STATIC && TWCfg<T, G, REV, STATIC>::NM >= 4 && ((BF && FIT_TT) || FIT_FT);
  static constexpr bool DX = BF && (SH ? FIT_TT : FIT_TF);
  using type = TWLdsT<T, G, REV, STATIC, DX, SH>;
};
template <typename T, class G, bool REV, bool STATIC = false>
using TWLds = typename TWPick<T, G, REV, STATIC>::type;

// W^T frags of the dX contraction for column tile ct, built into registers
// (same entries as build_wt_frags).
template <typename T, class G>
__device__ __forceinline__ void wt_frags_reg(const float* __restrict__ W, int ld, int L, int P, int ct,
                                             typename Eng<T>::frag (&wt)[G::NQS]) {
  using E = Eng<T>;
  const int lane = lane_id();
  const int c = 32 * ct + (lane & 31), h = lane >> 5;
#pragma unroll
  for (int qs = 0; qs < G::NQS; ++qs) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 16 * qs + 8 * h + i;
      float w = 0.f;
      if (e < G::NE && ct < G::CT) {
        const int hp = e % G::NHP, which = e / G::NHP;
        const int l = hp / G::PE, t = hp % G::PE;
        if (l < L && t < P) {
          const float x = w_entry(W, ld, l * P + t, c);
          const float xh = E::round(x);
          w = (E::NSPLIT == 2 && which == 2) ? (x - xh) : (E::NSPLIT == 2 ? xh : x);
        }
      }
      v[i] = w;
    }
    wt[qs] = E::pack(v);
  }
}

// ------------------------------------------------------------------ race_walk_tw
// Per chunk, wave w (bucket rows [R0, R0 + URP)), with the bank B[c][lr] of
// its rows (columns of the state-role values X, plus the mass column kept as
// a vector m) in registers:
//   dphi[lr][a] = sum_c B[lr][c] U_a[c] + m[lr] ue_a                       (inter)
//               + sum_{b in chunk, masked} phi_B,b[lr] (X_b . U_a + xe_b ue_a)  (intra)
//   forward walk (dPhi_Q): U = dO, ue = h den, xe = 1, then dphi /= den_a
//   reverse walk (dPhi_K): U = V,  ue = 1,     xe = h, X = g = dO / den
//   softmax, tanh backward of the wave's tables -> dPre (to LDS)
//   B[c][lr] += sum_b X_b[c] phi_B,b[lr],  m[lr] += sum_b phi_B,b[lr] xe_b
// and, at the top of the next chunk, dX = dPre . W for the wave's column
// tiles.  The masked intra scores are formed once per chunk by four waves
// and shared through LDS behind a workgroup barrier (where the stages fit;
// else each wave forms them).  Rows of the next chunk are staged into LDS by
// the whole workgroup at the end of the chunk (one barrier); X^T operands of
// the bank update come from the staged rows through transposing LDS loads
// (bf16; float32 I/O multiplies the rows by an identity operand).
template <typename T, class G, bool REV, int TG, bool STATIC = false>
__device__ __forceinline__ void tw_body(const TWArgs& a, TWLds<T, G, REV, STATIC>& S) {
  using C = TWCfg<T, G, REV, STATIC>;
  using SL = TWLds<T, G, REV, STATIC>;
  auto sb = [](int bb) { return SL::NSB == 2 ? bb : 0; };   // buffer of the AR, BR, UF rows
  using E = Eng<T>;
  using frag = typename E::frag;
  constexpr int R0 = TG * C::URP;
  constexpr int URP = C::URP, ATU = C::ATU;
  constexpr int DP1 = G::D + 1;
  constexpr int FS = C::FS, TSP = C::TSP;
  constexpr int EPC = C::EPC, CPR = C::CPR;
  using WT = WinTiles<G, R0, URP>;
  typedef T T4 __attribute__((ext_vector_type(4)));
  auto plain = [](int c) { return c; };
  const int lane = lane_id(), n = lane & 31, h = lane >> 5;
  const int w = TG;
  const int tid = threadIdx.x;
  const int64_t seg = blockIdx.x, bh = blockIdx.y;
  const int64_t s0 = seg * a.seg_tokens, s1 = min(a.N, s0 + a.seg_tokens);
  const int64_t nch = (s1 - s0 + WC - 1) / WC;
  const size_t rb = (size_t)bh * a.N;
  // bank rows: [d+1] per segment bank, or content rows [d] of the static bank
  constexpr int BS = STATIC ? G::D : DP1;
  const size_t bank_off = (STATIC ? (size_t)bh : (size_t)bh * a.nseg + seg) * G::LRP * BS;
  const T* Ag = static_cast<const T*>(a.A_src) + rb * G::D;
  const T* Bg = static_cast<const T*>(a.B_src) + rb * G::D;
  const T* Xg = static_cast<const T*>(a.X_src) + rb * G::D;
  const T* Ug = static_cast<const T*>(a.U_src) + rb * G::D;
  const float* den = a.den + rb;
  const float* hv = a.hvec + rb;
  T* dXg = static_cast<T*>(a.dX) + rb * G::D;
  const float beta2 = 2.f * a.beta;

  frag wt[C::NCTW][G::NQS];
#pragma unroll
  for (int j = 0; j < C::NCTW; ++j) wt_frags_reg<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, w + C::NM * j, wt[j]);
  // identity operands: lane (c, h), element i is 1 where kmap(s, h, i) == c
  frag idn[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = kmap(s, h, i) == n ? 1.f : 0.f;
    idn[s] = E::pack(v);
  }

  f32x16 acc[ATU][G::CT];
#pragma unroll
  for (int at = 0; at < ATU; ++at) {
    const size_t rowo = bank_off + (size_t)(R0 + 32 * at + n) * BS;
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[at][ct][v] = a.bank_in[rowo + 32 * ct + 8 * (v >> 2) + 4 * h + (v & 3)];
    if (h == 0)
      S.Mw[w][32 * at + n] = STATIC ? a.mass_in[(size_t)bh * G::LRP + R0 + 32 * at + n] : a.bank_in[rowo + G::D];
  }

  // ---- staging loads (chunk index clamped: loads never sit behind a branch)
  uint4 px[C::NPS], pu[C::NPS], pa[C::NPS], pb[C::NPS];
  float pd[C::NPS];
  float tk_h = 0.f, tk_d = 1.f;
  // PRE: this wave's tables' stored projections of the lane's token, both
  // roles: loaded with the staging loads, kept in registers from the staging
  constexpr int NSW = (WT::L1 - WT::L0) * G::PE;
  float qa[C::PRE ? NSW : 1], qb[C::PRE ? NSW : 1], ca[C::PRE ? NSW : 1], cb[C::PRE ? NSW : 1];
  const float* preAg = C::PRE ? a.preA_in + rb * G::NHP + WT::L0 * G::PE : nullptr;
  const float* preBg = C::PRE ? a.preB_in + rb * G::NHP + WT::L0 * G::PE : nullptr;
  auto load_stage = [&](int64_t k) {
    const int64_t t0 = chunk_t0<REV>(s0, nch, k < nch ? k : nch - 1);
#pragma unroll
    for (int i = 0; i < C::NPS; ++i) {
      const int idx = min(tid + C::NT * i, WC * CPR - 1);
      const int64_t row = min(t0 + idx / CPR, s1 - 1);
      const int cc = idx % CPR;
      if (!STATIC) px[i] = *reinterpret_cast<const uint4*>(Xg + row * G::D + cc * EPC);
      pu[i] = *reinterpret_cast<const uint4*>(Ug + row * G::D + cc * EPC);
      if (!C::PRE) pa[i] = *reinterpret_cast<const uint4*>(Ag + row * G::D + cc * EPC);
      if (!STATIC && !C::PRE) pb[i] = *reinterpret_cast<const uint4*>(Bg + row * G::D + cc * EPC);
      if (REV && !STATIC) pd[i] = den[row];
    }
    const int64_t row = min(t0 + n, s1 - 1);
    tk_h = hv[row];
    tk_d = den[row];
    if constexpr (C::PRE) {
#pragma unroll
      for (int j = 0; j < NSW; ++j) {
        qa[j] = preAg[row * G::NHP + j];
        qb[j] = preBg[row * G::NHP + j];
      }
    }
  };
  // ---- write the staged chunk k into buffer bb
  auto stage = [&](int64_t k, int bb) {
    const int64_t t0 = chunk_t0<REV>(s0, nch, k);
#pragma unroll
    for (int i = 0; i < C::NPS; ++i) {
      const int idx = tid + C::NT * i;
      if (idx < WC * CPR) {
        const int r = idx / CPR, cc = idx % CPR;
        const bool ok = t0 + r < s1;
        if constexpr (!C::PRE) {
          *reinterpret_cast<uint4*>(&S.AR[sb(bb)][r * FS + cc * EPC]) = pa[i];
          if (!STATIC) *reinterpret_cast<uint4*>(&S.BR[sb(bb)][r * FS + cc * EPC]) = pb[i];
        }
        // rows past the segment end are zero; only X = g = dO / den of the
        // reverse walk is converted (bf16: hi + lo parts), the rest is copied
        const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);
        const uint4 uv = ok ? pu[i] : zero4;
        uint4 xv = ok ? px[i] : zero4, xlv = zero4;
        if constexpr (REV && !STATIC) {
          const T* xe8 = reinterpret_cast<const T*>(&px[i]);
          const float sc = rcp(pd[i]);
          T xh[EPC], xl[EPC];
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            const float f = ok ? (float)xe8[e] * sc : 0.f;
            xh[e] = (T)f;
            xl[e] = (T)(f - (float)xh[e]);
          }
          xv = *reinterpret_cast<const uint4*>(xh);
          xlv = *reinterpret_cast<const uint4*>(xl);
        }
        // kmap frag order: column 16 q + 8 hh + e sits at 16 q + 8 (e / 4) + 4 hh + e % 4,
        // so a 16-byte chunk of bf16 goes out as two 8-byte halves
        const T* uu = reinterpret_cast<const T*>(&uv);
        const T* xh = reinterpret_cast<const T*>(&xv);
        const T* xl = reinterpret_cast<const T*>(&xlv);
#pragma unroll
        for (int g4 = 0; g4 < EPC / 4; ++g4) {
          const int col = cc * EPC + 4 * g4;
          const int q = col >> 4, o = col & 15, hh = o >> 3, ee = o & 7;
          const int pos = r * FS + 16 * q + 8 * (ee >> 2) + 4 * hh;
          *reinterpret_cast<T4*>(&S.UF[sb(bb)][pos]) = *reinterpret_cast<const T4*>(&uu[4 * g4]);
          if (!STATIC) *reinterpret_cast<T4*>(&S.XF[bb][0][pos]) = *reinterpret_cast<const T4*>(&xh[4 * g4]);
          if (C::XSPLIT) *reinterpret_cast<T4*>(&S.XF[bb][1][pos]) = *reinterpret_cast<const T4*>(&xl[4 * g4]);
        }
      }
    }
    if (tid < WC) {
      const bool ok = t0 + tid < s1;
      S.TK[bb][0][tid] = ok ? (REV ? tk_h : 1.f) : 0.f;        // xe
      S.TK[bb][1][tid] = ok ? (REV ? 1.f : tk_h * tk_d) : 0.f; // ue
      S.TK[bb][2][tid] = ok ? 1.f / tk_d : 0.f;                 // 1 / den
      if constexpr (C::TRB) {
        const float xe = ok ? (REV ? tk_h : 1.f) : 0.f;
        const T xh = (T)xe;
        S.XEB[bb][0][tid] = xh;
        S.XEB[bb][1][tid] = (T)(xe - (float)xh);
      }
    }
    if constexpr (C::PRE) {
#pragma unroll
      for (int j = 0; j < NSW; ++j) {
        ca[j] = qa[j];
        cb[j] = qb[j];
      }
    }
  };
  // ---- dPre of slot hp of this lane's token (chunk starting at t0) into buffer bb
  auto put_dpre = [&](int bb, int64_t t0, int hp, float x) {
    bb = SL::NDB == 2 ? bb : 0;
    if constexpr (SL::DXB) {
      T* r = S.DB[bb] + n * C::DBS;
      const T xh = (T)x;
      const T xl = (T)(x - (float)xh);
      r[hp] = xh;
      r[G::NHP + hp] = xl;
      r[2 * G::NHP + hp] = xh;
      if (a.dpre_out && t0 + n < s1) a.dpre_out[((size_t)bh * a.N + t0 + n) * G::NHP + hp] = x;
    } else {
      S.DP[bb][n * C::DPS + hp] = x;
    }
  };
  // ---- dX = dPre . W for chunk k (from DP[bb] / DB[bb]), this wave's column tiles
  auto dx_out = [&](int64_t k, int bb) {
    bb = SL::NDB == 2 ? bb : 0;
    const int64_t t0 = chunk_t0<REV>(s0, nch, k);
    frag bq[G::NQS];
    if constexpr (SL::DXB) {
      const T* r = S.DB[bb] + n * C::DBS + 8 * h;
#pragma unroll
      for (int qs = 0; qs < G::NQS; ++qs) bq[qs] = *reinterpret_cast<const frag*>(r + 16 * qs);
    } else {
      float dp[G::NHP];
#pragma unroll
      for (int i = 0; i < G::NHP; ++i) dp[i] = S.DP[bb][n * C::DPS + i];
      if (a.dpre_out && w == 0 && t0 + n < s1)
        store_dpre_half<G>(a.dpre_out + ((size_t)bh * a.N + t0 + n) * G::NHP, dp, h);
#pragma unroll
      for (int qs = 0; qs < G::NQS; ++qs) bq[qs] = dpre_frag<T, G>(dp, qs);
    }
#pragma unroll
    for (int j = 0; j < C::NCTW; ++j) {
      const int ct = w + C::NM * j;
      if (ct < G::CT) {
        f32x16 o = zero16();
#pragma unroll
        for (int qs = 0; qs < G::NQS; ++qs) E::mma(wt[j][qs], bq[qs], o);
        if (t0 + n < s1) store_tl_tile<T>(dXg + (t0 + n) * G::D, ct, o, 1.f);
      }
    }
  };

  // ---- intra-chunk scores of the chunk staged in buffer bb: sub-tile i =
  // (b rows 16 (i / 2) .., a columns 16 (i % 2) ..) by wave NM - 1 - i (mod
  // NM): mf[b][a] = X_b . U_a + xe_b ue_a, masked (b <= a forward, b >= a
  // reverse), on the 16 x 16 MFMA
  auto score_tiles = [&](int bb) {
    if constexpr (SL::SHSC) {
    const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (((C::NM - 1 - i) % C::NM + C::NM) % C::NM != TG) continue;
      const int bt = i >> 1, at2 = i & 1;
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
      const T* xr = S.XF[bb][0] + (16 * bt + l16) * FS + 8 * g4;
      const T* xl = S.XF[bb][C::NXS - 1] + (16 * bt + l16) * FS + 8 * g4;
      const T* ur = S.UF[sb(bb)] + (16 * at2 + l16) * FS + 8 * g4;
#pragma unroll
      for (int st = 0; st < G::D / 32; ++st) {
        const frag ub = *reinterpret_cast<const frag*>(ur + 32 * st);
        E::mma16(*reinterpret_cast<const frag*>(xr + 32 * st), ub, c);
        if (C::XSPLIT) E::mma16(*reinterpret_cast<const frag*>(xl + 32 * st), ub, c);
      }
      // lane (l16, g4) holds b = 16 bt + 4 g4 + r, a = 16 at2 + l16
      const int ta = 16 * at2 + l16, b0 = 16 * bt + 4 * g4;
      const float ue = S.TK[bb][1][ta];
      const f32x4 xe4 = *reinterpret_cast<const f32x4*>(&S.TK[bb][0][b0]);
      float m4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool keep = REV ? (b0 + r >= ta) : (b0 + r <= ta);
        const float m = c[r] + xe4[r] * ue;
        m4[r] = keep ? m : 0.f;
      }
      const int pos = (b0 & ~15) + 8 * ((b0 >> 2) & 1) + 4 * ((b0 >> 3) & 1);
      typename E::vec4 hv, lv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hv[r] = (T)m4[r];
        lv[r] = (T)(m4[r] - (float)hv[r]);
      }
      *reinterpret_cast<typename E::vec4*>(S.MFT[0] + ta * C::MS + pos) = hv;
      if (E::NSPLIT == 2) *reinterpret_cast<typename E::vec4*>(S.MFT[E::NSPLIT - 1] + ta * C::MS + pos) = lv;
    }
    }
  };

  if constexpr (C::PRE) {
    // projections come stored
  } else if constexpr (C::SPL > 1) {
    build_table_frags<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, S.Wf);
  } else {
    build_proj_frags<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, S.Wf);
  }
  if constexpr (SL::DXB) {
    // entries past 3 NHP are never written: zero (W^T is zero there too)
    for (int i = tid; i < SL::NDB * WC * C::DBS; i += C::NT) (&S.DB[0][0])[i] = (T)0.f;
  }
  load_stage(0);
  stage(0, 0);
  __syncthreads();
  float bsum = 0.f;

  for (int64_t k = 0; k < nch; ++k) {
    const int bb = (int)(k & 1);
    const int64_t t0 = chunk_t0<REV>(s0, nch, k);
    const bool valid = t0 + n < s1;
    // dX of chunk k - 1 (its dPre rows are complete since the last barrier),
    // then this wave's share of the chunk's intra scores
    if (k > 0) dx_out(k - 1, bb ^ 1);
    if constexpr (SL::SHSC) score_tiles(bb);
    // features of chunk k: output role (float32, kept), state role (rounded, to LDS)
    float preA[G::NHP], evA[G::NHP], phA[URP / 2];
    {
      if constexpr (C::PRE) {
#pragma unroll
        for (int hp = 0; hp < G::NHP; ++hp) preA[hp] = 0.f;
#pragma unroll
        for (int j = 0; j < NSW; ++j) preA[WT::L0 * G::PE + j] = ca[j];
      } else {
        frag xa[G::KD];
#pragma unroll
        for (int q = 0; q < G::KD; ++q) xa[q] = *reinterpret_cast<const frag*>(&S.AR[sb(bb)][n * FS + 16 * q + 8 * h]);
        if constexpr (C::SPL > 1) project_table<T, G, R0 / G::R>(S.Wf, xa, preA);
        else project_tiles<T, G, WT::PT0, WT::PT1>(S.Wf, xa, preA);
      }
      soft_assign_rows<G, R0, URP>(preA, beta2, a.L, evA, phA);
    }
    if constexpr (!STATIC) {
      float pre[G::NHP], evB[G::NHP], phB[URP / 2];
      if constexpr (C::PRE) {
#pragma unroll
        for (int hp = 0; hp < G::NHP; ++hp) pre[hp] = 0.f;
#pragma unroll
        for (int j = 0; j < NSW; ++j) pre[WT::L0 * G::PE + j] = cb[j];
      } else {
        frag xb[G::KD];
#pragma unroll
        for (int q = 0; q < G::KD; ++q) xb[q] = *reinterpret_cast<const frag*>(&S.BR[sb(bb)][n * FS + 16 * q + 8 * h]);
        if constexpr (C::SPL > 1) project_table<T, G, R0 / G::R>(S.Wf, xb, pre);
        else project_tiles<T, G, WT::PT0, WT::PT1>(S.Wf, xb, pre);
      }
      soft_assign_rows<G, R0, URP>(pre, beta2, a.L, evB, phB, valid);   // zero rows past the segment end
      T* pt = S.PhiBT[w];
      if constexpr (C::TRB) {
        // token row n: bucket rows 8 g + 4 h .. + 3 of each 32-row tile
#pragma unroll
        for (int at = 0; at < ATU; ++at)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            T4 v4;
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] = (T)phB[16 * at + 4 * g + j];
            *reinterpret_cast<T4*>(pt + n * C::RS + 32 * at + 8 * g + 4 * h) = v4;
          }
      } else {
#pragma unroll
        for (int at = 0; at < ATU; ++at)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int lr = 32 * at + 8 * (v >> 2) + 4 * h + (v & 3);
            pt[lr * TSP + n] = (T)phB[16 * at + v];
          }
      }
    }
    wave_lds_sync();

    // inter: bank . U_a (U exact in T), and the intra scores
    // mf[b][a] = X_b . U_a (+ xe_b ue_a below), masked (b <= a forward, b >= a
    // reverse); one read of each U fragment serves both
    f32x16 dp[ATU];
#pragma unroll
    for (int at = 0; at < ATU; ++at) dp[at] = zero16();
    // per-wave intra scores (without shared scores): mf[b][a] = X_b . U_a
    constexpr bool OWN = !STATIC && !SL::SHSC;
    f32x16 mf = zero16();
    {
      const T* uf = S.UF[sb(bb)] + n * FS + 8 * h;
      const T* xf = S.XF[bb][0] + n * FS + 8 * h;
      const T* xl = S.XF[bb][C::NXS - 1] + n * FS + 8 * h;
      // operands of step q + 1 are loaded before the MFMAs of step q
      frag ubq[2], xfq[2], xlq[2];
      auto ldq = [&](int q) {
        const int sl = q & 1;
        ubq[sl] = *reinterpret_cast<const frag*>(uf + 16 * q);
        xfq[sl] = OWN ? *reinterpret_cast<const frag*>(xf + 16 * q) : E::zero();
        xlq[sl] = (OWN && C::XSPLIT) ? *reinterpret_cast<const frag*>(xl + 16 * q) : E::zero();
      };
      ldq(0);
#pragma unroll
      for (int q = 0; q < G::KD; ++q) {
        const frag ub = ubq[q & 1], xfv = xfq[q & 1], xlv = xlq[q & 1];
        if (q + 1 < G::KD) ldq(q + 1);
#pragma unroll
        for (int at = 0; at < ATU; ++at) {
          float v8[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v8[i] = acc[at][q >> 1][8 * (q & 1) + i];
          if (C::BANK_LO && E::NSPLIT == 2) {
            frag hi, lo;
            E::split(v8, hi, lo);
            E::mma(hi, ub, dp[at]);
            E::mma(lo, ub, dp[at]);
          } else {
            E::mma(E::pack(v8), ub, dp[at]);
          }
        }
        if (OWN) E::mma(xfv, ub, mf);
        if (OWN && C::XSPLIT) E::mma(xlv, ub, mf);
      }
    }
    const float ue = S.TK[bb][1][n];
    if constexpr (OWN) {
      // xe of the lane's 16 score rows (four runs of 4 consecutive tokens),
      // read whether masked or not: a load under the mask compiles to a
      // branch and a wait per element
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 xe4 = *reinterpret_cast<const f32x4*>(&S.TK[bb][0][8 * g + 4 * h]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = 4 * g + j, tb = 8 * g + 4 * h + j;
          const bool keep = REV ? (tb >= n) : (tb <= n);
          const float m = mf[v] + xe4[j] * ue;
          mf[v] = keep ? m : 0.f;
        }
      }
    }
    // the chunk's shared intra scores are complete
    if constexpr (SL::SHSC) __syncthreads();
    // mass term and intra part: dp[lr][a] += m[lr] ue_a + sum_b phi_B,b[lr] mf[b][a]
    {
      const T* pt = S.PhiBT[w];
#pragma unroll
      for (int at = 0; at < ATU; ++at) {
#pragma unroll
        for (int v = 0; v < 16; ++v) dp[at][v] += S.Mw[w][32 * at + 8 * (v >> 2) + 4 * h + (v & 3)] * ue;
      }
#pragma unroll
      for (int s = 0; s < (STATIC ? 0 : 2); ++s) {
        frag mh, ml;
        if constexpr (SL::SHSC) {
          const T* mr = S.MFT[0] + n * C::MS + 16 * s + 8 * h;
          mh = *reinterpret_cast<const frag*>(mr);
          ml = *reinterpret_cast<const frag*>(S.MFT[E::NSPLIT - 1] + n * C::MS + 16 * s + 8 * h);
        } else {
          float m8[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) m8[i] = mf[8 * s + i];
          E::split(m8, mh, ml);
        }
#pragma unroll
        for (int at = 0; at < ATU; ++at) {
          frag af;
          if constexpr (C::TRB) {
            af = load_kcol_tr(pt, C::RS, 16 * s, 32 * at, plain);
          } else {
            const T* r = pt + (32 * at + n) * TSP + 16 * s + 4 * h;
            const T4 lo4 = *reinterpret_cast<const T4*>(r);
            const T4 hi4 = *reinterpret_cast<const T4*>(r + 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              af[i] = lo4[i];
              af[4 + i] = hi4[i];
            }
          }
          E::mma(af, mh, dp[at]);
          if (E::NSPLIT == 2) E::mma(af, ml, dp[at]);
        }
      }
    }
    // softmax, tanh backward of the wave's tables -> dPre (forward walk: dphi = dp / den)
    {
      const float sc = REV ? 1.f : S.TK[bb][2][n];
      float dphi[URP / 2];
#pragma unroll
      for (int at = 0; at < ATU; ++at)
#pragma unroll
        for (int v = 0; v < 16; ++v) dphi[16 * at + v] = dp[at][v] * sc;
      float dpre[G::NHP], bterm = 0.f;
#pragma unroll
      for (int i = 0; i < G::NHP; ++i) dpre[i] = 0.f;
      if constexpr (C::SPL == 1) {
        assign_backward_rows<G, R0, URP>(phA, dphi, preA, a.beta, dpre, bterm);
        if (valid && h == 0) bsum += bterm;
        if (h == 0) {
#pragma unroll
          for (int hp = WT::L0 * G::PE; hp < WT::L1 * G::PE; ++hp) put_dpre(bb, t0, hp, dpre[hp]);
        }
      } else {
        // split table: exchange the sums with the table's other waves (TG0 ..
        // TG0 + SPL - 1), add them in the same order in every one of them,
        // then dU_t = A_t - s E[v_t] with E[v_t] = tanh(beta u_t) from the
        // soft assignment; each lane half takes the hyperplanes it evaluated
        // there, and the pairs of hyperplanes (t, t + 1) are dealt to the
        // table's waves in turn (pair t / 2 to wave TG0 + (t / 2) % SPL), which
        // write their dPre and add their dbeta terms
        constexpr int TG0 = TG - TG % C::SPL;
        constexpr int l = R0 / G::R;
        float part[1 + G::PE];
        assign_partials_split<G, R0>(phA, dphi, part);
        if (h == 0) {
#pragma unroll
          for (int i = 0; i <= G::PE; ++i) S.XS[w][i][n] = part[i];
        }
        __syncthreads();
        auto table_sum = [&](int i) {
          float v = S.XS[TG0][i][n];
#pragma unroll
          for (int j = 1; j < C::SPL; ++j) v += S.XS[TG0 + j][i][n];
          return v;
        };
        const float s = table_sum(0);
#pragma unroll
        for (int t = 0; t < G::PE; t += 2) {
          if ((t / 2) % C::SPL != TG - TG0) continue;
          const bool pair = t + 1 < G::PE;
          const int tt = pair ? t + h : t;
          float uu, s2;
          tanh_sech2((pair && h) ? preA[l * G::PE + t + 1] : preA[l * G::PE + t], uu, s2);
          const float du = table_sum(1 + tt) - s * evA[l * G::PE + t];
          if (pair || h == 0) {
            bterm += uu * du;
            put_dpre(bb, t0, l * G::PE + tt, a.beta * du * s2);
          }
        }
        if (valid) bsum += bterm;
      }
    }
    // rows of chunk k + 1: loaded here rather than at the top of the chunk
    // (their registers are not live through the features and readout)
    load_stage(k + 1);
    __builtin_amdgcn_sched_barrier(0);
    // bank update: B[c][lr] += sum_b X_b[c] phi_B,b[lr]; X^T tiles (lane = column,
    // registers = tokens in kmap order) from X rows times the identity
    if constexpr (!STATIC) {
      const T* pt = S.PhiBT[w];
      frag pb[2][ATU];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int at = 0; at < ATU; ++at) {
          if constexpr (C::TRB) {
            pb[s][at] = load_kcol_tr(pt, C::RS, 16 * s, 32 * at, plain);
          } else {
            const T* r = pt + (32 * at + n) * TSP + 16 * s + 4 * h;
            const T4 lo4 = *reinterpret_cast<const T4*>(r);
            const T4 hi4 = *reinterpret_cast<const T4*>(r + 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pb[s][at][i] = lo4[i];
              pb[s][at][4 + i] = hi4[i];
            }
          }
        }
      if constexpr (std::is_same<T, bf16>::value) {
        // X^T operands straight from the staged rows through transposing LDS
        // loads, issued PF steps ahead of their MFMAs; step j: part j / (2 CT),
        // column tile (j / 2) % CT, token half j % 2
        constexpr int NSTEP = C::NXS * G::CT * 2, PF = 4;
        auto ldx = [&](int j) {
          return load_kcol_tr(S.XF[bb][j / (2 * G::CT)], FS, 16 * (j & 1), 32 * ((j >> 1) % G::CT), kmap_run_pos);
        };
        frag xq[PF];
#pragma unroll
        for (int j = 0; j < PF; ++j) xq[j] = ldx(j);
#pragma unroll
        for (int j = 0; j < NSTEP; ++j) {
          const frag xa = xq[j % PF];
          if (j + PF < NSTEP) xq[j % PF] = ldx(j + PF);
#pragma unroll
          for (int at = 0; at < ATU; ++at) E::mma(xa, pb[j & 1][at], acc[at][(j >> 1) % G::CT]);
        }
      } else {
#pragma unroll
        for (int sp = 0; sp < C::NXS; ++sp) {
          const T* xf = S.XF[bb][sp] + n * FS + 8 * h;
#pragma unroll
          for (int ct = 0; ct < G::CT; ++ct) {
            f32x16 xt = zero16();
            E::mma(*reinterpret_cast<const frag*>(xf + 16 * (2 * ct)), idn[0], xt);
            E::mma(*reinterpret_cast<const frag*>(xf + 16 * (2 * ct + 1)), idn[1], xt);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              float x8[8];
#pragma unroll
              for (int i = 0; i < 8; ++i) x8[i] = xt[8 * s + i];
              const frag xa = E::pack(x8);
#pragma unroll
              for (int at = 0; at < ATU; ++at) E::mma(xa, pb[s][at], acc[at][ct]);
            }
          }
        }
      }
      // mass: bf16, lane (n, h) sums the tokens of its bank-update operands
      // (16 s + kmap(0, h, i)); float32: lane half h sums tokens 16 h .. 16 h
      // + 15 of row 32 at + n
#pragma unroll
      for (int at = 0; at < ATU; ++at) {
        float sm = 0.f;
        if constexpr (C::TRB) {
          // xe as hi + lo (forward walk: 0 or 1, exact in bf16, no lo part)
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            sm = dot8_bf16(pb[s][at], load_kmap8(S.XEB[bb][0], 16 * s, h), sm);
            if (REV) sm = dot8_bf16(pb[s][at], load_kmap8(S.XEB[bb][1], 16 * s, h), sm);
          }
        } else {
          const T* r = pt + (32 * at + n) * TSP + 16 * h;
#pragma unroll
          for (int t = 0; t < 16; ++t) sm += (float)r[t] * S.TK[bb][0][16 * h + t];
        }
        sm += xor32(sm);
        if (h == 0) S.Mw[w][32 * at + n] += sm;
      }
    }
    // staging of chunk k + 1
    if (k + 1 < nch) stage(k + 1, bb ^ 1);
    __syncthreads();
  }
  dx_out(nch - 1, (int)((nch - 1) & 1));
  if (a.dbeta_part) {
    bsum = wave_sum(bsum);
    if (lane == 0) a.dbeta_part[((size_t)bh * a.nseg + seg) * C::NM + w] = bsum;
  }
}

template <typename T, class G, bool REV, bool STATIC, int TG>
__device__ __forceinline__ void tw_dispatch(int w, const TWArgs& a, TWLds<T, G, REV, STATIC>& S) {
  if (w == TG) {
    tw_body<T, G, REV, TG, STATIC>(a, S);
  } else if constexpr (TG + 1 < TWCfg<T, G, REV, STATIC>::NM) {
    tw_dispatch<T, G, REV, STATIC, TG + 1>(w, a, S);
  }
}

template <typename T, class G, bool REV, bool STATIC = false>
__global__ __launch_bounds__((TWCfg<T, G, REV, STATIC>::NT)) void race_walk_tw(TWArgs a) {
  __shared__ TWLds<T, G, REV, STATIC> S;
  tw_dispatch<T, G, REV, STATIC, 0>(threadIdx.x >> 6, a, S);
}

// ------------------------------------------------------------------ small kernels
// dbeta = sum of the per-wave shares, in a fixed order (one workgroup of 256).
static __global__ void race_dbeta_finalize(const float* __restrict__ part, int64_t n, float* __restrict__ out) {
  __shared__ float red[256];
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int m = 128; m > 0; m >>= 1) {
    if ((int)threadIdx.x < m) red[threadIdx.x] += red[threadIdx.x + m];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0];
}

// h_t = -(dO_t . O_t) / den_t for every token when the caller hands over O:
// 16 lanes per token row, one 16-byte chunk each.
template <typename T, int D>
__global__ __launch_bounds__(256) void race_h_from_o(const T* __restrict__ dO, const T* __restrict__ O,
                                                     const float* __restrict__ den, float* __restrict__ h,
                                                     int64_t total) {
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int LPT = D / EPC;   // lanes per token (16 bf16 / 32 f32 for d = 128)
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tok = gid / LPT;
  const int part = (int)(gid % LPT);
  float s = 0.f;
  if (tok < total) {
    const uint4 a = *reinterpret_cast<const uint4*>(dO + tok * D + part * EPC);
    const uint4 b = *reinterpret_cast<const uint4*>(O + tok * D + part * EPC);
    const T* x = reinterpret_cast<const T*>(&a);
    const T* y = reinterpret_cast<const T*>(&b);
#pragma unroll
    for (int e = 0; e < EPC; ++e) s += (float)x[e] * (float)y[e];
  }
#pragma unroll
  for (int m = LPT / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, 64);
  if (tok < total && part == 0) h[tok] = -s / den[tok];
}


// Exclusive scan over segments (forward: banks before each segment; reverse:
// banks after it), one thread per (bh, bank element).
static __global__ void race_seg_scan(const float* __restrict__ part, float* __restrict__ out, int nseg, int per, int BH,
                              int reverse) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)BH * per) return;
  const int64_t bh = idx / per, rem = idx % per;
  float run = 0.f;
  // unrolled so that several segment loads are in flight at once
#pragma unroll 8
  for (int k = 0; k < nseg; ++k) {
    const int s = reverse ? nseg - 1 - k : k;
    const size_t o = ((size_t)bh * nseg + s) * per + rem;
    const float v = part[o];
    out[o] = run;
    run += v;
  }
}

}  // namespace race
