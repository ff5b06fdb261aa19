// Causal prefix walks in the readout layout (slides frame "Causality is a
// prefix update of the same statistics", paper Algorithm 2; reading notes
// section 2.6), one cooperative workgroup per (segment, batch x head).
//
// A workgroup walks its segment in 32-token chunks.  It has two kinds of
// waves:
//   feature waves  soft-assign the token rows of the chunk AHEAD (projection
//                  on MFMA, tanh and sigmoid products on VALU) into a
//                  double-buffered LDS stage, each for one role (output or
//                  state) and one window of bucket rows, and keep the running
//                  bucket mass of their window;
//   bank waves     hold one 32-column slice of the bucket bank
//                  S[lr][c] (lr over all L*R buckets) in MFMA accumulators and
//                  do every contraction of the current chunk.
// One workgroup barrier per chunk hands a stage from the feature waves to the
// bank waves, so soft bucketing (VALU) of chunk k+1 overlaps the bank
// contractions (MFMA) of chunk k on every SIMD.
//
// Per chunk, with Phi_A the output-role and Phi_B the state-role features,
// X the state-role values and S, m the bank and mass before the chunk:
//   y   = Phi_A S + tril(Phi_A Phi_B^T) X          (inter + intra part)
//   den = Phi_A m + rowsum tril(Phi_A Phi_B^T)
//   S  += Phi_B^T X,  m += Phi_B^T 1
// (tril keeps j <= t on forward walks and j >= t on reverse walks.)
// Modes:
//   W_SEGSUM  bank of every segment: S = Phi_K^T V, m = Phi_K^T 1
//   W_GSUM    gradient bank of every segment: Phi_Q^T g, Phi_Q^T h
//             with g = dO / den, h = -(dO . O) / den, formed as
//             (Phi_Q / den)^T dO and (Phi_Q / den)^T (h den): the state-role
//             features absorb 1 / den and X = dO stays exact
//   W_FWD     O = y / den from the segment's starting bank; writes den
//   W_H       h = -(dO . y) / den^2 (y = O den), without O
//   W_DV      reverse walk, output role K, state role Q / den, X = dO:
//             dV_j = sum_{t >= j} (phi_K,j . phi_Q,t) g_t
// Static modes (the non-causal layer for bucket counts whose whole bank does
// not fit one wave): every token reads one fixed bank per (batch, head) (the
// segment index is ignored), with no intra-chunk term and no bank update,
// so only output-role feature waves run:
//   W_FWD_ST  O = Phi_Q content / Phi_Q mass
//   W_H_ST    Den = Phi_Q mass and h = -(dO . Phi_Q content) / Den^2, both written
//   W_DV_ST   dV = Phi_K dcontent
#pragma once
#include "race_device.hpp"

namespace race {

constexpr int WC = 32;   // tokens per chunk

enum { W_SEGSUM = 0, W_GSUM = 1, W_FWD = 2, W_H = 3, W_DV = 4, W_FWD_ST = 5, W_H_ST = 6, W_DV_ST = 7 };

struct WArgs {
  const void* A_src;      // output-role token rows (FWD, H: Q; DV: K)
  const void* B_src;      // state-role token rows (SEGSUM, FWD, H: K; GSUM, DV: Q)
  const void* X_src;      // state-role values (V; GSUM, DV: dO)
  const void* dO;         // H: dO rows of the output role
  void* out;              // FWD: O (NULL: only Den is written); DV: dV
  float* bank_out;        // SEGSUM, GSUM: [BH][nseg][LRP][d+1]
  const float* bank_in;   // FWD, H, DV: [BH][nseg][LRP][d+1], bank before (after, DV) the segment;
                          // static modes: content [BH][LRP][d]
  const float* mass_in;   // static modes: mass [BH][LRP]
  const float* den;       // [BH][N]: GSUM, H, DV
  float* den_out;         // FWD: [BH][N]
  const float* hvec;      // GSUM: h [BH][N]
  float* h_out;           // H: [BH][N]
  // causal backward, when set: the projections W x that GSUM makes of its
  // state role (Q) and DV of its output role (K), float32 [BH][N][NHP] (slot
  // l PE + t), kept for the transposed walks; with split tables DV's
  // state-role waves read GSUM's (preB_in) instead of projecting Q
  float* pre_out;
  const float* preB_in;
  Tables W;
  float beta;
  int L, P;
  int64_t N;
  int64_t seg_tokens;
  int nseg;
};

// Largest divisor of n that is <= cap.
__host__ __device__ constexpr int div_le(int n, int cap) {
  int best = 1;
  for (int d = 1; d <= cap; ++d)
    if (n % d == 0) best = d;
  return best;
}

template <typename T, class G, int MODE>
struct RWCfg {
  static constexpr bool STATIC = MODE >= W_FWD_ST;          // one fixed bank, no update
  static constexpr int BM = STATIC ? MODE - 3 : MODE;       // the walk's readout mode
  static constexpr bool HAS_A = BM >= W_FWD;                // an output role is read out
  static constexpr bool REV = BM == W_DV;                   // walk from the segment end
  static constexpr int ROLES = (HAS_A && !STATIC) ? 2 : 1;  // feature roles
  static constexpr int NWIN = div_le(G::LRP / 32, ROLES == 2 ? 2 : 4);   // row windows per role
  static constexpr int WROWS = G::LRP / NWIN;
  // bf16, one table per feature window: each table gets its own projection
  // tile (hi + lo rows), so every window projects exactly one tile (shared
  // 8-slot tiles would give windows whose table straddles two tiles twice
  // the work)
  static constexpr bool TABLE_TILES = std::is_same<T, bf16>::value && WROWS == G::R && G::PE <= 8;
  static constexpr int NF = ROLES * NWIN;                   // feature waves
  static constexpr int NM = G::CT;                          // bank waves
  static constexpr int NT = 64 * (NF + NM);
  static constexpr bool MASS = (BM == W_SEGSUM || BM == W_GSUM || BM == W_FWD) && !STATIC;   // mass updates
  static constexpr bool MBUF = MASS || (STATIC && BM != W_DV);   // a bucket mass is kept in LDS
  static constexpr bool DEN = BM == W_FWD || (STATIC && BM == W_H);   // feature waves form Phi_A mass
  // bf16: the mass is also kept as bf16 hi + lo rows (after the float32 rows
  // of mbuf), so that Phi_A . mass runs on v_dot2
  static constexpr bool DENB = DEN && std::is_same<T, bf16>::value;
  // GSUM, DV: the state role's features are divided by its token's den, so
  // that with X = dO the bank sums phi_Q g^T (and, GSUM, with mass weights
  // h den, phi_Q h)
  static constexpr bool PHIDEN = (BM == W_GSUM || BM == W_DV) && !STATIC;
  // GSUM (state role) and DV (output role) store the projections they make
  static constexpr bool PRE_OUT_A = BM == W_DV && !STATIC;
  static constexpr bool PRE_OUT_B = BM == W_GSUM && !STATIC;
  // projection slots of one window: its tables, or the one table it is part of
  static constexpr int NSW = (WROWS >= G::R ? WROWS / G::R : 1) * G::PE;
  // split tables (the sets whose transposed walks read stored projections):
  // DV's state-role waves load GSUM's stored W Q into the registers that
  // otherwise hold the Q row (FPF floats per row fragment), so reading them
  // costs no registers
  static constexpr int FPF = (int)(sizeof(typename Eng<T>::frag) / sizeof(float));
  static constexpr bool PRE_B = BM == W_DV && !STATIC && G::R > 32 && (NSW + FPF - 1) / FPF <= G::KD;
  static constexpr bool XROWS = !STATIC;                    // bank waves read X rows
  // frag-ordered feature row per token and bank-wave X tile row (elements):
  // with bf16, rows 12 dwords apart (mod 64 banks) keep both the 16-byte row
  // reads and the transposing loads (4 rows x 8 dwords per 16 lanes) free
  // of bank conflicts
  static constexpr int FR = G::KL * 16 + (std::is_same<T, bf16>::value ? 24 : 8);
  static constexpr int TS = WC + 8;             // transposed feature row per bucket (elements)
  static constexpr int XSP = 32 + (std::is_same<T, bf16>::value ? 24 : 8);
  // bf16: the state-role features are kept in token-major rows only (PhiB)
  // and read transposed (bank-update operands, bucket masses) with
  // transposing LDS loads; float32 keeps a transposed copy (PhiBT)
  static constexpr bool TRLOAD = std::is_same<T, bf16>::value;
  static constexpr bool ROWS_B = !STATIC && (HAS_A || TRLOAD);   // PhiB rows are written
  // The float32 bank enters the readout rounded once to the MFMA type (its
  // relative error 2^-9 matches the rounding of the bf16 outputs); with
  // BANK_LO the rounding residual is contracted as well.
  static constexpr bool BANK_LO = false;
};

// Bucket mass of row `row` into buffer `buf` of mbuf (float32 rows [2][LRP],
// then with BF the bf16 hi and lo rows [2][2][LRP]).
template <typename T, class G, bool BF>
__device__ __forceinline__ void put_mass(float* mbuf, int buf, int row, float v) {
  mbuf[buf * G::LRP + row] = v;
  if constexpr (BF) {
    T* mb = reinterpret_cast<T*>(mbuf + 2 * G::LRP) + (2 * buf) * G::LRP + row;
    const T vh = (T)v;
    mb[0] = vh;
    mb[G::LRP] = (T)(v - (float)vh);
  }
}

// First token of the k-th chunk in walk order.
template <bool REV>
__device__ __forceinline__ int64_t chunk_t0(int64_t s0, int64_t nch, int64_t k) {
  return s0 + (REV ? (nch - 1 - k) : k) * WC;
}

// ------------------------------------------------------------------ feature waves
// Soft-assign the 32 rows of one chunk for bucket rows [R0, R0 + WROWS) and
// publish them: output role as frag-ordered rows (B operands of the readout),
// state role as frag-ordered rows and transposed rows (bank update), plus
// the mass bookkeeping of the window.  RBM: the wave's role when fixed at
// compile time (0 output, 1 state), -1 when taken from role_b (PRE_B walks
// instantiate the two roles separately).
template <typename T, class G, int MODE, int R0, int RBM = -1>
__device__ __forceinline__ void rw_feature_window(const WArgs& a, const typename Eng<T>::frag* __restrict__ Wf,
                                                  const typename Eng<T>::frag (&xf)[G::KD], float hv, float dv,
                                                  bool role_b_rt, int64_t t0, int64_t s1, int b, int fw,
                                                  T* __restrict__ PhiA,
                                                  T* __restrict__ PhiB, T* __restrict__ PhiBT,
                                                  float* __restrict__ mbuf, float* __restrict__ dpart,
                                                  float* __restrict__ hw, int win) {
  using C = RWCfg<T, G, MODE>;
  using E = Eng<T>;
  using frag = typename E::frag;
  constexpr int WROWS = C::WROWS;
  constexpr int NQ = WROWS / 16;
  using WT = WinTiles<G, R0, WROWS>;
  const int lane = lane_id(), n = lane & 31, h = lane >> 5;
  const int64_t tok = t0 + n;
  const bool valid = tok < s1;
  const bool role_b = RBM < 0 ? role_b_rt : RBM == 1;
  T* hwb = reinterpret_cast<T*>(hw + C::NF * WC);
  float pre[G::NHP], ev[G::NHP], phi[WROWS / 2];
  static_assert((WT::L1 - WT::L0) * G::PE == C::NSW, "window slots");
  if constexpr (C::PRE_B && RBM == 1) {
    // the stored projections of the window's tables, carried in xf
    typedef float fv __attribute__((ext_vector_type(C::FPF)));
#pragma unroll
    for (int hp = 0; hp < G::NHP; ++hp) pre[hp] = 0.f;
#pragma unroll
    for (int j = 0; j < C::NSW; ++j) pre[WT::L0 * G::PE + j] = __builtin_bit_cast(fv, xf[j / C::FPF])[j % C::FPF];
  } else {
    if constexpr (C::TABLE_TILES) project_table<T, G, R0 / G::R>(Wf, xf, pre);
    else project_tiles<T, G, WT::PT0, WT::PT1>(Wf, xf, pre);
    if ((role_b ? C::PRE_OUT_B : C::PRE_OUT_A) && a.pre_out && h == 0 && valid) {
      // the slots of the window's tables
      float* dst = a.pre_out + ((size_t)blockIdx.y * a.N + tok) * G::NHP + WT::L0 * G::PE;
#pragma unroll
      for (int j = 0; j < C::NSW; ++j) dst[j] = pre[WT::L0 * G::PE + j];
    }
  }
  // tokens past the segment end: zero rows; state role of GSUM, DV: / den
  soft_assign_rows<G, R0, WROWS, C::PRE_B && RBM == 1>(pre, 2.f * a.beta, a.L, ev, phi, valid,
                                                       (C::PHIDEN && role_b) ? 1.f / dv : 1.f);
  frag fq[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) fq[q] = tl_frag<T, WROWS>(phi, q);
  if (!role_b) {
    T* dst = PhiA + b * WC * C::FR + n * C::FR + (R0 / 16) * 16 + h * 8;
#pragma unroll
    for (int q = 0; q < NQ; ++q) *reinterpret_cast<frag*>(dst + 16 * q) = fq[q];
    if (C::DEN) {
      // den (inter part) over this window: rounded phi_A . mass before the
      // chunk (static modes: the fixed mass, kept in buffer 1)
      const int mb = C::STATIC ? 1 : (b ^ 1);
      float d = 0.f;
      if constexpr (C::DENB) {
        const T* mh = reinterpret_cast<const T*>(mbuf + 2 * G::LRP) + (2 * mb) * G::LRP + R0;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          d = dot8_bf16(fq[q], load_kmap8(mh, 16 * q, h), d);
          d = dot8_bf16(fq[q], load_kmap8(mh + G::LRP, 16 * q, h), d);
        }
      } else {
        const float* m = mbuf + mb * G::LRP + R0;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int i = 0; i < 8; ++i) d += (float)fq[q][i] * m[kmap(q, h, i)];
      }
      d += xor32(d);
      if (h == 0) dpart[(b * C::NWIN + win) * WC + n] = d;
    }
    return;
  }
  if constexpr (C::STATIC) return;   // static modes have no state role
  if constexpr (C::ROWS_B) {
    T* dst = PhiB + b * WC * C::FR + n * C::FR + (R0 / 16) * 16 + h * 8;
#pragma unroll
    for (int q = 0; q < NQ; ++q) *reinterpret_cast<frag*>(dst + 16 * q) = fq[q];
  }
  if constexpr (!C::TRLOAD) {
    T* bt = PhiBT + b * G::LRP * C::TS;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) bt[(R0 + kmap(q, h, i)) * C::TS + n] = fq[q][i];
  }
  if (C::MASS) {
    if (C::BM == W_GSUM && h == 0) {
      const float wv = valid ? hv * dv : 0.f;
      hw[fw * WC + n] = wv;
      if constexpr (C::TRLOAD) {
        // the weights as bf16 hi + lo for the mass sums on v_dot2
        const T wh = (T)wv;
        hwb[(2 * fw) * WC + n] = wh;
        hwb[(2 * fw + 1) * WC + n] = (T)(wv - (float)wh);
      }
    }
    wave_lds_sync();
    // mass after the chunk = mass before + column sums of the rounded phi_B
    // (GSUM: weighted by h)
    if constexpr (C::TRLOAD) {
      // lane (n, h) sums the tokens kmap(s, h, i) of bucket row R0 + 32 at + n;
      // the two halves then add their sums
      const T* rows = PhiB + b * WC * C::FR;
#pragma unroll
      for (int at = 0; at < WROWS / 32; ++at) {
        float sm = 0.f;
#pragma unroll
        for (int sidx = 0; sidx < 2; ++sidx) {
          const frag v = load_kcol_tr(rows, C::FR, 16 * sidx, R0 + 32 * at, kmap_run_pos);
          if constexpr (C::BM == W_GSUM) {
            sm = dot8_bf16(v, load_kmap8(hwb + (2 * fw) * WC, 16 * sidx, h), sm);
            sm = dot8_bf16(v, load_kmap8(hwb + (2 * fw + 1) * WC, 16 * sidx, h), sm);
          } else {
            sm = dot8_bf16(v, E::ones(), sm);
          }
        }
        sm += xor32(sm);
        const int row = R0 + 32 * at + n;
        if (h == 0) put_mass<T, G, C::DENB>(mbuf, b, row, mbuf[(b ^ 1) * G::LRP + row] + sm);
      }
    } else {
      const T* bt = PhiBT + b * G::LRP * C::TS;
#pragma unroll
      for (int r = 0; r < cdiv(WROWS, 64); ++r) {
        const int row = R0 + 64 * r + lane;
        if (64 * r + lane < WROWS) {
          const T* src = bt + row * C::TS;
          float s = 0.f;
#pragma unroll
          for (int t = 0; t < WC; ++t) s += (C::BM == W_GSUM) ? (float)src[t] * hw[fw * WC + t] : (float)src[t];
          mbuf[b * G::LRP + row] = mbuf[(b ^ 1) * G::LRP + row] + s;
        }
      }
    }
  }
}

template <typename T, class G, int MODE, int WI>
__device__ __forceinline__ void rw_feature_dispatch(int win, const WArgs& a, const typename Eng<T>::frag* Wf,
                                                    const typename Eng<T>::frag (&xf)[G::KD], float hv, float dv,
                                                    bool role_b,
                                                    int64_t t0, int64_t s1, int b, int fw, T* PhiA, T* PhiB,
                                                    T* PhiBT, float* mbuf, float* dpart, float* hw) {
  using C = RWCfg<T, G, MODE>;
  if (win == WI) {
    if constexpr (C::PRE_B) {
      if (role_b)
        rw_feature_window<T, G, MODE, WI * C::WROWS, 1>(a, Wf, xf, hv, dv, role_b, t0, s1, b, fw, PhiA, PhiB,
                                                        PhiBT, mbuf, dpart, hw, WI);
      else
        rw_feature_window<T, G, MODE, WI * C::WROWS, 0>(a, Wf, xf, hv, dv, role_b, t0, s1, b, fw, PhiA, PhiB,
                                                        PhiBT, mbuf, dpart, hw, WI);
    } else {
      rw_feature_window<T, G, MODE, WI * C::WROWS>(a, Wf, xf, hv, dv, role_b, t0, s1, b, fw, PhiA, PhiB, PhiBT,
                                                   mbuf, dpart, hw, WI);
    }
  } else if constexpr (WI + 1 < C::NWIN) {
    rw_feature_dispatch<T, G, MODE, WI + 1>(win, a, Wf, xf, hv, dv, role_b, t0, s1, b, fw, PhiA, PhiB, PhiBT, mbuf,
                                            dpart, hw);
  }
}

// ------------------------------------------------------------------ the walk
template <typename T, class G, int MODE>
__global__ __launch_bounds__((RWCfg<T, G, MODE>::NT)) void race_walk_rw(WArgs a) {
  using C = RWCfg<T, G, MODE>;
  using E = Eng<T>;
  using frag = typename E::frag;
  constexpr int NS = E::NSPLIT;
  constexpr int FR = C::FR, TS = C::TS, XSP = C::XSP;
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  constexpr int CPR = 32 / EPC;              // 16-byte chunks per 32-column row slice
  constexpr int XIT = WC * CPR / 64;         // row-slice loads per lane
  constexpr int DP1 = G::D + 1;

  __shared__ frag Wf[(C::TABLE_TILES ? G::LMAX : G::NPT) * G::KD * 64];
  __shared__ __attribute__((aligned(16))) T PhiA[C::HAS_A ? 2 * WC * FR : 8];
  __shared__ __attribute__((aligned(16))) T PhiB[C::ROWS_B ? 2 * WC * FR : 8];
  __shared__ __attribute__((aligned(16))) T PhiBT[(C::TRLOAD || C::STATIC) ? 8 : 2 * G::LRP * TS];
  __shared__ __attribute__((aligned(16))) T Xs[C::NM * WC * XSP];
  __shared__ float mbuf[C::MBUF ? (C::DENB ? 4 : 2) * G::LRP : 1];
  __shared__ float dpart[C::DEN ? 2 * C::NWIN * WC : 1];
  __shared__ float hpart[C::BM == W_H ? 2 * C::NM * WC : 1];
  // GSUM: mass weights h den per feature wave and token, then (bf16) the
  // same weights as hi + lo parts
  __shared__ float hw[C::BM == W_GSUM ? 2 * C::NF * WC : 1];

  const int64_t seg = blockIdx.x, bh = blockIdx.y;
  const int lane = lane_id(), n = lane & 31, h = lane >> 5, w = threadIdx.x >> 6;
  const int64_t s0 = seg * a.seg_tokens, s1 = min(a.N, s0 + a.seg_tokens);
  const int64_t nch = (s1 - s0 + WC - 1) / WC;
  const size_t rb = (size_t)bh * a.N;
  // bank rows: [d+1] per segment bank, or content rows [d] of the static bank
  constexpr int BS = C::STATIC ? G::D : DP1;
  const size_t bank_off = (C::STATIC ? (size_t)bh : (size_t)bh * a.nseg + seg) * G::LRP * BS;
  const bool is_f = w < C::NF;
  // feature wave: role and window; bank wave: column tile
  const bool role_b = C::STATIC ? false : (C::HAS_A ? (w >= C::NWIN) : true);
  const int win = w % C::NWIN;
  const int ct = w - C::NF;

  if constexpr (C::TABLE_TILES) build_table_frags<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, Wf);
  else build_proj_frags<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, Wf);
  if ((C::MASS && is_f && role_b) || (C::STATIC && C::MBUF && is_f)) {
    for (int r = lane; r < C::WROWS; r += 64) {
      const int row = win * C::WROWS + r;
      put_mass<T, G, C::DENB>(mbuf, 1, row,
                              C::STATIC          ? a.mass_in[(size_t)bh * G::LRP + row]
                              : (C::BM == W_FWD) ? a.bank_in[bank_off + (size_t)row * DP1 + G::D]
                                                 : 0.f);
    }
  }

  if (is_f) {
    // ---------------------------------------------------------------- feature waves
    const T* src = static_cast<const T*>(role_b ? a.B_src : a.A_src) + rb * G::D;
    const float* hsrc = a.hvec + rb;
    const float* dsrc = a.den + rb;
    frag xa[G::KD], xb[G::KD];
    float ha = 0.f, hb = 0.f, da = 1.f, db = 1.f;   // h and den of the wave's token
    // PRE_B state role: the window's stored projections W Q
    const float* psrc = C::PRE_B ? a.preB_in + rb * G::NHP + (win * C::WROWS / G::R) * G::PE : nullptr;
    // Loads are issued for every iteration (the chunk index clamped to the
    // last one) so no prefetch sits behind a branch: the compiler then waits
    // only for the rows a projection actually consumes.
    auto load = [&](int64_t k, frag(&xf)[G::KD], float& hv, float& dv) {
      const int64_t t0 = chunk_t0<C::REV>(s0, nch, k < nch ? k : nch - 1);
      const int64_t row = min(t0 + n, s1 - 1);
      if (C::BM == W_GSUM) hv = hsrc[row];
      if (C::PHIDEN && role_b) dv = dsrc[row];
      if (C::PRE_B && role_b) {
        typedef float fv __attribute__((ext_vector_type(C::FPF)));
#pragma unroll
        for (int q = 0; q < (C::NSW + C::FPF - 1) / C::FPF; ++q) {
          fv v;
#pragma unroll
          for (int i = 0; i < C::FPF; ++i) v[i] = q * C::FPF + i < C::NSW ? psrc[row * G::NHP + q * C::FPF + i] : 0.f;
          xf[q] = __builtin_bit_cast(frag, v);
        }
      } else {
        load_row_frags_nb<T, G>(src + row * G::D, xf);
      }
    };
    auto feat = [&](int64_t k, const frag(&xf)[G::KD], float hv, float dv) {
      const int64_t t0 = chunk_t0<C::REV>(s0, nch, k);
      rw_feature_dispatch<T, G, MODE, 0>(win, a, Wf, xf, hv, dv, role_b, t0, s1, (int)(k & 1), w, PhiA, PhiB,
                                         PhiBT, mbuf, dpart, hw);
    };
    load(0, xa, ha, da);
    load(1, xb, hb, db);
    __syncthreads();
    feat(0, xa, ha, da);
    __syncthreads();
    // iteration k: features of chunk k + 1 (rows in xb), rows of chunk k + 2 -> xa
    for (int64_t k = 0; k < nch; k += 2) {
      load(k + 2, xa, ha, da);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 1 < nch) feat(k + 1, xb, hb, db);
      __syncthreads();
      if (k + 1 >= nch) break;
      load(k + 3, xb, hb, db);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 2 < nch) feat(k + 2, xa, ha, da);
      __syncthreads();
    }
    if (C::MASS && role_b && (C::BM == W_SEGSUM || C::BM == W_GSUM)) {
      const int fb = (int)((nch - 1) & 1);
      for (int r = lane; r < C::WROWS; r += 64) {
        const int row = win * C::WROWS + r;
        a.bank_out[bank_off + (size_t)row * DP1 + G::D] = mbuf[fb * G::LRP + row];
      }
    }
    return;
  }

  // ------------------------------------------------------------------ bank waves
  f32x16 st[G::AT];
#pragma unroll
  for (int at = 0; at < G::AT; ++at) {
    if (C::BM == W_SEGSUM || C::BM == W_GSUM) {
      st[at] = zero16();
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = 32 * at + 8 * (v >> 2) + 4 * h + (v & 3);
        st[at][v] = a.bank_in[bank_off + (size_t)lr * BS + 32 * ct + n];
      }
    }
  }
  T* xs = Xs + ct * WC * XSP;
  const T* Xg = static_cast<const T*>(a.X_src) + rb * G::D + 32 * ct;
  const T* dOg = (C::BM == W_H) ? static_cast<const T*>(a.dO) + rb * G::D + 32 * ct : nullptr;
  const float* den = a.den + rb;

  // prefetch registers: X row slices, dO slices (H)
  uint4 xr[XIT];
  typename E::vec4 dor[4];
  auto prefetch = [&](int64_t k) {
    const int64_t t0 = chunk_t0<C::REV>(s0, nch, k);
    if constexpr (C::XROWS) {
#pragma unroll
      for (int it = 0; it < XIT; ++it) {
        const int flat = it * 64 + lane;
        const int64_t row = min(t0 + flat / CPR, s1 - 1);
        xr[it] = *reinterpret_cast<const uint4*>(Xg + row * G::D + (flat % CPR) * EPC);
      }
    }
    if (C::BM == W_H) {
      const int64_t row = min(t0 + n, s1 - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dor[j] = *reinterpret_cast<const typename E::vec4*>(dOg + row * G::D + 8 * j + 4 * h);
    }
  };
  prefetch(0);
  __syncthreads();   // projection frags, initial mass
  __syncthreads();   // stage of chunk 0

  float dn_prev = 1.f;   // static H: Den of the previous chunk's token (ct = 0 wave)
  for (int64_t k = 0; k < nch; ++k) {
    const int b = (int)(k & 1);
    const int64_t t0 = chunk_t0<C::REV>(s0, nch, k);
    const int64_t tok = t0 + n;
    const bool valid = tok < s1;
    // H: finish h of the previous chunk from the column-slice partial dots
    if (C::BM == W_H && ct == 0 && k > 0 && h == 0) {
      const int64_t pt = chunk_t0<C::REV>(s0, nch, k - 1) + n;
      if (pt < s1) {
        float s = 0.f;
#pragma unroll
        for (int m = 0; m < C::NM; ++m) s += hpart[((b ^ 1) * C::NM + m) * WC + n];
        const float dd = C::STATIC ? dn_prev : den[pt];
        a.h_out[rb + pt] = -s / (dd * dd);
      }
    }
    // stage this chunk's X slice (rows past the segment end are zero)
#pragma unroll
    for (int it = 0; it < (C::XROWS ? XIT : 0); ++it) {
      const int flat = it * 64 + lane;
      const int row = flat / CPR, ch = flat % CPR;
      const bool ok = t0 + row < s1;
      *reinterpret_cast<uint4*>(xs + row * XSP + ch * EPC) = ok ? xr[it] : make_uint4(0, 0, 0, 0);
    }
    typename E::vec4 dcur[4];
    if (C::BM == W_H) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dcur[j] = dor[j];
    }
    prefetch(k + 1 < nch ? k + 1 : k);
    __builtin_amdgcn_sched_barrier(0);
    wave_lds_sync();
    // X frags, k over tokens by kmap: lane (c, h) holds X[kmap(s, h, i)][c]
    frag xk[2];
    if constexpr (!C::XROWS) {
      // static modes read no X rows
    } else if constexpr (C::TRLOAD) {
      auto plain = [](int c) { return c; };
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        xk[s] = load_kcol_tr(xs, XSP, 16 * s, 0, plain);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          xk[s][i] = xs[kmap(s, h, i) * XSP + n];
        }
    }

    if constexpr (C::HAS_A) {
      const T* pA = PhiA + b * WC * FR + n * FR + h * 8;
      const T* pB = PhiB + b * WC * FR + n * FR + h * 8;
      f32x16 y = zero16(), sc = zero16();
      // feature frags are loaded two K16 steps ahead of their MFMAs
      frag fa[3], fb[3];
#pragma unroll
      for (int q = 0; q < 2 && q < G::KL; ++q) {
        fa[q] = *reinterpret_cast<const frag*>(pA + 16 * q);
        if (!C::STATIC) fb[q] = *reinterpret_cast<const frag*>(pB + 16 * q);
      }
#pragma unroll
      for (int q = 0; q < G::KL; ++q) {
        if (q + 2 < G::KL) {
          fa[(q + 2) % 3] = *reinterpret_cast<const frag*>(pA + 16 * (q + 2));
          if (!C::STATIC) fb[(q + 2) % 3] = *reinterpret_cast<const frag*>(pB + 16 * (q + 2));
        }
        float v8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v8[i] = st[q >> 1][8 * (q & 1) + i];
        if (C::BANK_LO && NS == 2) {
          frag hi, lo;
          E::split(v8, hi, lo);
          E::mma(hi, fa[q % 3], y);
          E::mma(lo, fa[q % 3], y);
        } else {
          E::mma(E::pack(v8), fa[q % 3], y);
        }
        if (!C::STATIC) E::mma(fb[q % 3], fa[q % 3], sc);
      }
      // intra: sc[tok_b][tok_a] = phi_B . phi_A, kept for tok_b <= tok_a (>= on reverse walks)
      float dsum = 0.f;
      if constexpr (!C::STATIC) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int tb = 8 * (v >> 2) + 4 * h + (v & 3);
          const bool keep = C::REV ? (tb >= n) : (tb <= n);
          sc[v] = keep ? sc[v] : 0.f;
          dsum += sc[v];
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          float s8[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) s8[i] = sc[8 * s + i];
          const frag sb = E::pack(s8);
          E::mma(xk[s], sb, y);
        }
      }
      // static H: Den of this chunk's tokens from the feature waves' parts
      if (C::STATIC && C::BM == W_H && ct == 0 && h == 0) {
        float dn = 0.f;
#pragma unroll
        for (int p = 0; p < C::NWIN; ++p) dn += dpart[(b * C::NWIN + p) * WC + n];
        dn_prev = dn;
        if (valid) a.den_out[rb + tok] = dn;
      }
      // y: lane (tok, h) holds columns 32 ct + 8 j + 4 h + kk
      if (C::BM == W_FWD || C::BM == W_DV) {
        float scale = 1.f;
        if (C::BM == W_FWD) {
          dsum += xor32(dsum);
          float dn = dsum;
#pragma unroll
          for (int p = 0; p < C::NWIN; ++p) dn += dpart[(b * C::NWIN + p) * WC + n];
          scale = 1.f / dn;
          if (a.den_out && ct == 0 && h == 0 && valid) a.den_out[rb + tok] = dn;
        }
        // stage the 32 x 32 output tile in the X tile, then store 64-byte row pieces
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          typename E::vec4 o;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) o[kk] = (T)(y[4 * j + kk] * scale);
          *reinterpret_cast<typename E::vec4*>(xs + n * XSP + 8 * j + 4 * h) = o;
        }
        wave_lds_sync();
        // FWD with out == NULL: Den only (the backward rebuilding its state)
        if (a.out) {
          T* og = static_cast<T*>(a.out) + rb * G::D + 32 * ct;
#pragma unroll
          for (int it = 0; it < XIT; ++it) {
            const int flat = it * 64 + lane;
            const int row = flat / CPR, ch = flat % CPR;
            const uint4 v = *reinterpret_cast<const uint4*>(xs + row * XSP + ch * EPC);
            if (t0 + row < s1) *reinterpret_cast<uint4*>(og + (t0 + row) * G::D + ch * EPC) = v;
          }
        }
      } else if (C::BM == W_H) {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) part += (float)dcur[j][kk] * y[4 * j + kk];
        part += xor32(part);
        if (h == 0) hpart[(b * C::NM + ct) * WC + n] = part;
      }
    }
    // bank update: S[lr][c] += sum_tok Phi_B[tok][lr] X[tok][c]
    if constexpr (!C::STATIC) {
      const T* bt = PhiBT + b * G::LRP * TS;
      typedef T T4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        frag af[G::AT];
#pragma unroll
        for (int at = 0; at < G::AT; ++at) {
          if constexpr (C::TRLOAD) {
            af[at] = load_kcol_tr(PhiB + b * WC * FR, FR, 16 * s, 32 * at, kmap_run_pos);
          } else {
            const T* r = bt + (32 * at + n) * TS + 16 * s + 4 * h;
            const T4 lo4 = *reinterpret_cast<const T4*>(r);
            const T4 hi4 = *reinterpret_cast<const T4*>(r + 8);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              af[at][i] = lo4[i];
              af[at][4 + i] = hi4[i];
            }
          }
        }
#pragma unroll
        for (int at = 0; at < G::AT; ++at) {
          E::mma(af[at], xk[s], st[at]);
        }
      }
    }
    __syncthreads();
  }
  if (C::BM == W_H && ct == 0 && h == 0) {
    const int b = (int)((nch - 1) & 1);
    const int64_t pt = chunk_t0<C::REV>(s0, nch, nch - 1) + n;
    if (pt < s1) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < C::NM; ++m) s += hpart[(b * C::NM + m) * WC + n];
      const float dd = C::STATIC ? dn_prev : den[pt];
      a.h_out[rb + pt] = -s / (dd * dd);
    }
  }
  if (C::BM == W_SEGSUM || C::BM == W_GSUM) {
#pragma unroll
    for (int at = 0; at < G::AT; ++at)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = 32 * at + 8 * (v >> 2) + 4 * h + (v & 3);
        a.bank_out[bank_off + (size_t)lr * DP1 + 32 * ct + n] = st[at][v];
      }
  }
}

}  // namespace race
