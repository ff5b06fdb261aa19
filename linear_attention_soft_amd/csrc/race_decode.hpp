// Recurrent decode step: the causal RACE layer as a fixed-size recurrent
// state (slides frame "Causality is a prefix update of the same statistics",
// paper Algorithm 2; reading notes section 2.6).  The state of every
// (batch, head) is its bucket bank after the tokens seen so far: content
// [LRP][d] and mass [LRP], float32 (the same layout as the non-causal state).
// For each new token t, in order: the key is added first, then the query
// reads (the token sees itself):
//   content += phi(K_t) V_t^T,  mass += phi(K_t)
//   O_t = sum_l phi(Q_t) content / sum_l phi(Q_t) mass
// One workgroup of NT = d * NG threads per (batch, head): thread (column c,
// row group g) keeps bank rows [g * LRP / NG, (g + 1) * LRP / NG) of column c
// in registers for all new tokens; NG gives at least 256 threads and at most
// 1024, and about 16 bank rows per thread in between.  Projections, tanh, sigmoids and the soft
// assignments are float32 and are not rounded.
#pragma once
#include "race_device.hpp"

namespace race {

struct DArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* content;   // [BH][LRP][d], updated in place
  float* mass;      // [BH][LRP], updated in place
  Tables W;
  float beta;
  int L, P;
  int64_t N;        // new tokens per (batch, head)
  int dr;           // elements per Q, K, V, O row (the caller's d, at most D; W.ld is the same)
};

template <class G>
struct DecCfg {
  static constexpr int lo = 256 / G::D, hi = 1024 / G::D, want = G::LRP / 16;
  static constexpr int NG = want < lo ? lo : (want > hi ? hi : want);   // row groups per column
  static constexpr int NT = G::D * NG;                                  // threads per (batch, head)
};

template <typename T, class G>
__global__ __launch_bounds__((DecCfg<G>::NT)) void race_decode(DArgs a) {
  constexpr int D = G::D, LRP = G::LRP;
  constexpr int NG = DecCfg<G>::NG;
  constexpr int DEC_NT = DecCfg<G>::NT;
  constexpr int RPT = LRP / NG;            // bank rows per thread
  static_assert(DEC_NT % 64 == 0 && LRP % NG == 0, "thread layout");
  constexpr int TPH = 4;                   // threads per projection dot product
  static_assert(2 * G::NHP * TPH <= DEC_NT, "projection threads");
  __shared__ float xs[3][D];               // q, k, v of the current token
  __shared__ float sg[2][2][G::NHP];       // sigma(+-2 beta u) per role and hyperplane
  __shared__ float ph[2][LRP];             // soft assignments of q and k
  __shared__ float ms[LRP];                // mass
  __shared__ float num[NG][D];             // partial numerators
  __shared__ float red[DEC_NT / 64];       // per-wave partial denominators

  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t bh = blockIdx.x;
  const int c = tid % D, g = tid / D;
  float* content = a.content + (size_t)bh * LRP * D;
  float* mass = a.mass + (size_t)bh * LRP;
  const int dr = a.dr;
  const T* src[3] = {static_cast<const T*>(a.Q) + (size_t)bh * a.N * dr,
                     static_cast<const T*>(a.K) + (size_t)bh * a.N * dr,
                     static_cast<const T*>(a.V) + (size_t)bh * a.N * dr};
  T* out = static_cast<T*>(a.O) + (size_t)bh * a.N * dr;

  float bank[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) bank[i] = content[(size_t)(g * RPT + i) * D + c];
  for (int lr = tid; lr < LRP; lr += DEC_NT) ms[lr] = mass[lr];
  const float beta2 = 2.f * a.beta;
  // projection thread: (role, hyperplane, quarter of d)
  const int prole = tid / (G::NHP * TPH), php = (tid / TPH) % G::NHP, pq = tid % TPH;
  const int pl = php / G::PE, pt = php % G::PE;
  const bool pok = tid < 2 * G::NHP * TPH && pl < a.L && pt < a.P;
  const float* pw = a.W.at(bh) + (size_t)(pok ? pl * a.P + pt : 0) * a.W.ld;

  for (int64_t t = 0; t < a.N; ++t) {
    for (int i = tid; i < 3 * D; i += DEC_NT) {
      const int e = i % D;
      xs[i / D][e] = e < dr ? (float)src[i / D][t * dr + e] : 0.f;   // columns past dr are zero
    }
    __syncthreads();
    // projections: TPH consecutive lanes split d, then tanh and the sigmoid pair
    if (tid < 2 * G::NHP * TPH) {
      float s = 0.f;
      if (pok)
        for (int e = pq; e < dr; e += TPH) s += pw[e] * xs[prole][e];
#pragma unroll
      for (int m = TPH / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, 64);
      if (pq == 0) {
        float sp, sm;
        sigmoid_pair(beta2 * tanh_f(s), sp, sm);
        sg[prole][0][php] = sp;
        sg[prole][1][php] = sm;
      }
    }
    __syncthreads();
    // soft assignments phi_r = prod_t sigma(2 beta u_t v_{r,t})
    for (int j = tid; j < 2 * LRP; j += DEC_NT) {
      const int role = j / LRP, lr = j % LRP;
      const int l = lr / G::R, r = lr % G::R;
      float p = 0.f;
      if (l < a.L && l < G::LMAX) {
        p = 1.f;
#pragma unroll
        for (int tt = 0; tt < G::PE; ++tt) p *= sg[role][((r >> tt) & 1) ? 0 : 1][l * G::PE + tt];
      }
      ph[role][lr] = p;
    }
    __syncthreads();
    // key first, then the query reads the updated bank
    const float vc = xs[2][c];
    float nacc = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int lr = g * RPT + i;
      bank[i] += ph[1][lr] * vc;
      nacc += ph[0][lr] * bank[i];
    }
    num[g][c] = nacc;
    float dacc = 0.f;
    for (int lr = tid; lr < LRP; lr += DEC_NT) {
      ms[lr] += ph[1][lr];
      dacc += ph[0][lr] * ms[lr];
    }
    dacc = wave_sum(dacc);
    if (lane == 0) red[tid >> 6] = dacc;
    __syncthreads();
    if (g == 0) {
      float nn = 0.f;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) nn += num[gg][c];
      float den = 0.f;
#pragma unroll
      for (int k = 0; k < DEC_NT / 64; ++k) den += red[k];
      if (c < dr) out[t * dr + c] = (T)(nn / den);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) content[(size_t)(g * RPT + i) * D + c] = bank[i];
  for (int lr = tid; lr < LRP; lr += DEC_NT) mass[lr] = ms[lr];
}

}  // namespace race
