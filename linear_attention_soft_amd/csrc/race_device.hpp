// Device building blocks of the gfx950 RACE attention kernels.
//
// Lane layouts (CDNA4, 64-wide waves).  Every contraction runs on the
// 32x32 MFMA: v_mfma_f32_32x32x16_bf16 for bf16 I/O and eight
// v_mfma_f32_32x32x2_f32 for float32 I/O.  A "K16 step" contracts 16
// logical k indices; lane l = 32*h + n holds 8 of them for row/column n and
// half h.  The accumulator of a 32x32 tile puts element (m, n) in lane
// n + 32*((m/4)%2), register (m%4) + 4*(m/8).
//
// Token-major vectors ("TLAYOUT"): a per-token vector x of length M
// (M a multiple of 32) is held by the 64 lanes of a wave for 32 tokens:
// lane (tok, h) owns x[32*a + 8*j + 4*h + k] in register 16*a + 4*j + k.
// This is exactly the accumulator layout of a C^T[m][tok] tile, and read
// eight registers at a time it is a K16-step B operand whose logical index
// (h, i) of step q is  kmap(q, h, i) = 16*q + 8*(i/4) + 4*h + (i%4).
// Constant A operands that meet such a B operand are built with the same
// kmap, so no data moves between the MFMA that produces a TLAYOUT vector and
// the MFMA that consumes it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace race {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ constexpr int kmap(int q, int h, int i) {
  return 16 * q + 8 * (i >> 2) + 4 * h + (i & 3);
}

// ---------------------------------------------------------------- MFMA engines
template <typename T> struct Eng;

template <> struct Eng<bf16> {
  using frag = bf16x8;          // 8 bf16 per lane: one K16 step
  using vec4 = bf16x4;
  static constexpr int NSPLIT = 2;   // float operands are split hi + lo
  static constexpr int HPT = 8;      // hyperplanes per projection tile (hi and lo rows)
  __device__ __forceinline__ static void mma(const frag& a, const frag& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // 16x16 tile, K32 step: lane l holds k = 8*(l/16) + i of row / column l%16;
  // the accumulator holds element (m, n) in lane n + 16*(m/4), register m%4.
  __device__ __forceinline__ static void mma16(const frag& a, const frag& b, f32x4& c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag pack(const float* v) {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (bf16)v[i];
    return f;
  }
  __device__ __forceinline__ static void split(const float* v, frag& hi, frag& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bf16 x = (bf16)v[i];
      hi[i] = x;
      lo[i] = (bf16)(v[i] - (float)x);
    }
  }
  __device__ __forceinline__ static float round(float x) { return (float)(bf16)x; }
  __device__ __forceinline__ static frag ones() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (bf16)1.0f;
    return f;
  }
  __device__ __forceinline__ static frag zero() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (bf16)0.0f;
    return f;
  }
};

template <> struct Eng<float> {
  using frag = f32x8;           // 8 floats per lane: one K16 step = 8 MFMAs
  using vec4 = f32x4;
  static constexpr int NSPLIT = 1;
  static constexpr int HPT = 16;
  __device__ __forceinline__ static void mma(const frag& a, const frag& b, f32x16& c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[i], c, 0, 0, 0);
  }
  // 16x16 tile, K32 step (eight K4 MFMAs; element i of lane l is k = 8*(l/16) + i).
  __device__ __forceinline__ static void mma16(const frag& a, const frag& b, f32x4& c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag pack(const float* v) {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = v[i];
    return f;
  }
  __device__ __forceinline__ static void split(const float* v, frag& hi, frag& lo) {
    hi = pack(v);
    lo = hi;
  }
  __device__ __forceinline__ static float round(float x) { return x; }
  __device__ __forceinline__ static frag ones() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = 1.0f;
    return f;
  }
  __device__ __forceinline__ static frag zero() {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = 0.0f;
    return f;
  }
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ---------------------------------------------------------------- elementwise math
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh for any finite x: t = exp(-2|x|) in (0, 1], tanh|x| = (1 - t)/(1 + t).
__device__ __forceinline__ float tanh_f(float x) {
  float e = __expf(-2.f * fabsf(x));
  float t = (1.f - e) * rcp(1.f + e);
  return copysignf(t, x);
}

// tanh(x) and its derivative 1 - tanh(x)^2 = 4 e / (1 + e)^2 with e =
// exp(-2|x|), both to a few ulp of their own size: forming 1 - u^2 from a
// rounded u = tanh(x) near +-1 would lose the digits the derivative keeps.
__device__ __forceinline__ void tanh_sech2(float x, float& u, float& s2) {
  const float e = __expf(-2.f * fabsf(x));
  const float r = rcp(1.f + e);
  u = copysignf((1.f - e) * r, x);
  s2 = 4.f * e * r * r;
}

// sigma(z) and sigma(-z) without overflow for any finite z.
__device__ __forceinline__ void sigmoid_pair(float z, float& sp, float& sm) {
  float e = __expf(-fabsf(z));
  float p = rcp(1.f + e);   // sigma(|z|)
  float q = e * p;          // sigma(-|z|)
  bool pos = z >= 0.f;
  sp = pos ? p : q;
  sm = pos ? q : p;
}

// c + sum_i a[i] b[i] over 8 bf16 pairs, two products per v_dot2_f32_bf16
// (bf16 products are exact in float32)
__device__ __forceinline__ float dot8_bf16(const bf16x8& a, const bf16x8& b, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), c, false);
  return c;
}

// Eight bf16 values of a row kept in natural order at positions kmap(q, h, i)
// (two runs of four: q16 + 4 h and q16 + 8 + 4 h), as one operand.
__device__ __forceinline__ bf16x8 load_kmap8(const bf16* row, int q16, int h) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(row + q16 + 4 * h);
  const bf16x4 b = *reinterpret_cast<const bf16x4*>(row + q16 + 8 + 4 * h);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The two 32-lane halves of a wave exchanged in one VALU instruction
// (v_permlane32_swap): with both operands x it returns lanes 0-31 of x in
// every half (first) and lanes 32-63 of x in every half (second).
struct HalfPair { float lo, hi; };
__device__ __forceinline__ HalfPair halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Value of the same lane in the other half of the wave.
__device__ __forceinline__ float xor32(float v) {
  const HalfPair p = halves(v);
  return (threadIdx.x & 32) ? p.lo : p.hi;
}

// Projection tables: float32 [L][P][ld] shared by every head (hstride 0), or
// [H][L][P][ld] with one set per head (hstride L * P * ld).  Sequence bh of a
// [B][H] batch is head bh % H.  ld is the caller's head dim, at most the
// kernel's: columns at or past it read as zero (their token columns are zero
// too, so they add nothing to a projection).
struct Tables {
  const float* W;
  int64_t hstride;
  int H;
  int ld;
  __device__ __forceinline__ const float* at(int64_t bh) const { return W + (size_t)(bh % H) * hstride; }
};

// Entry (row, c) of a table set with row pitch ld (zero past ld).
__device__ __forceinline__ float w_entry(const float* __restrict__ W, int ld, int row, int c) {
  return c < ld ? W[(size_t)row * ld + c] : 0.f;
}

// ---------------------------------------------------------------- geometry
// Compile-time geometry of one kernel instance.
//   D     head dim (multiple of 32)
//   PE    hyperplanes per table used in-kernel, max(P, 3)
//   LRP   bucket rows, L * 2^PE rounded up to a multiple of 32
template <typename T, int D_, int PE_, int LRP_>
struct Geo {
  static constexpr int D = D_;
  static constexpr int PE = PE_;
  static constexpr int R = 1 << PE_;
  static constexpr int LRP = LRP_;
  static constexpr int LMAX = LRP_ / (1 << PE_) > 0 ? LRP_ / (1 << PE_) : 1;  // table slots
  static constexpr int NHP = LMAX * PE_;                       // hyperplane slots
  static constexpr int HPT = Eng<T>::HPT;
  static constexpr int NPT = cdiv(NHP, HPT);                   // projection tiles
  static constexpr int KD = D_ / 16;                           // K16 steps over d
  static constexpr int CT = D_ / 32;                           // 32-column tiles of d
  static constexpr int AT = LRP_ / 32;                         // 32-row tiles of buckets
  static constexpr int KL = LRP_ / 16;                         // K16 steps over buckets
  static constexpr int NE = (Eng<T>::NSPLIT == 2 ? 3 : 1) * NHP; // dX contraction entries
  static constexpr int NQS = cdiv(NE, 16);                     // K16 steps of the dX MFMA
  static_assert(D_ % 32 == 0, "d must be a multiple of 32");
  static_assert(LRP_ % 32 == 0, "LRP must be a multiple of 32");
  static_assert(PE_ >= 3 && PE_ <= 8, "3 <= PE <= 8");
  static_assert((1 << PE_) <= LRP_, "R must fit in LRP");
};

// ---------------------------------------------------------------- constant operands
// Projection A operand: rows are hyperplane "slots" (bf16: 8 hi rows then 8 lo
// rows per tile; f32: 16 rows), duplicated in both row halves so every lane
// ends with all pre-activations of its token; columns follow the plain map
// c = 16*q + 8*h + i of the token's row loads.
//
// float32 I/O keeps the plain rows instead, Wr[hp][c] (hp = l * PE + t, zero
// for l >= L or t >= P), in the same buffer: its projection is accumulated in
// float64 (project_rows_f64).
template <typename T, class G>
__device__ void build_proj_frags(const float* __restrict__ W, int ld, int L, int P,
                                 typename Eng<T>::frag* __restrict__ Wf) {
  using E = Eng<T>;
  if constexpr (std::is_same<T, float>::value) {
    static_assert(G::NHP * G::D <= G::NPT * G::KD * 64 * 8, "plain rows fit the operand buffer");
    float* Wr = reinterpret_cast<float*>(Wf);
    for (int idx = threadIdx.x; idx < G::NHP * G::D; idx += blockDim.x) {
      const int hp = idx / G::D, c = idx % G::D;
      const int l = hp / G::PE, t = hp % G::PE;
      Wr[idx] = (l < L && t < P) ? w_entry(W, ld, l * P + t, c) : 0.f;
    }
    return;
  }
  for (int idx = threadIdx.x; idx < G::NPT * G::KD * 64; idx += blockDim.x) {
    const int lane = idx & 63;
    const int q = (idx >> 6) % G::KD;
    const int pt = (idx >> 6) / G::KD;
    const int row = lane & 31, h = lane >> 5;
    const int rho = 4 * (row >> 3) + (row & 3);
    int hp, part;
    if (E::NSPLIT == 2) { hp = 8 * pt + (rho & 7); part = rho >> 3; }
    else                { hp = 16 * pt + rho;      part = 0; }
    const int l = hp / G::PE, t = hp % G::PE;
    const bool ok = (hp < G::NHP) && (l < L) && (t < P);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ok ? w_entry(W, ld, l * P + t, 16 * q + 8 * h + i) : 0.f;
    typename E::frag hi, lo;
    E::split(v, hi, lo);
    Wf[idx] = part ? lo : hi;
  }
}

// Projection A operand with one tile per table: tile l holds the PE
// hyperplanes of table l (bf16: rows t then the lo parts at 8 + t; f32: rows
// t), rows past PE zero, duplicated in both row halves as above.
template <typename T, class G>
__device__ void build_table_frags(const float* __restrict__ W, int ld, int L, int P,
                                  typename Eng<T>::frag* __restrict__ Wt) {
  using E = Eng<T>;
  static_assert(G::PE <= (E::NSPLIT == 2 ? 8 : 16), "one tile per table");
  static_assert(!std::is_same<T, float>::value, "float32 I/O projects from plain rows");
  for (int idx = threadIdx.x; idx < G::LMAX * G::KD * 64; idx += blockDim.x) {
    const int lane = idx & 63;
    const int q = (idx >> 6) % G::KD;
    const int l = (idx >> 6) / G::KD;
    const int row = lane & 31, h = lane >> 5;
    const int rho = 4 * (row >> 3) + (row & 3);
    const int t = E::NSPLIT == 2 ? (rho & 7) : rho;
    const int part = E::NSPLIT == 2 ? (rho >> 3) : 0;
    const bool ok = (t < G::PE) && (l < L) && (t < P);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ok ? w_entry(W, ld, l * P + t, 16 * q + 8 * h + i) : 0.f;
    typename E::frag hi, lo;
    E::split(v, hi, lo);
    Wt[idx] = part ? lo : hi;
  }
}

// pre[l * PE + t] = W^(l)_t . x for table l only (tile l of build_table_frags);
// other slots are 0.
template <typename T, class G, int l>
__device__ __forceinline__ void project_table(const typename Eng<T>::frag* __restrict__ Wt,
                                              const typename Eng<T>::frag (&xf)[G::KD], float (&pre)[G::NHP]) {
  using E = Eng<T>;
  const int lane = lane_id();
#pragma unroll
  for (int hp = 0; hp < G::NHP; ++hp) pre[hp] = 0.f;
  f32x16 acc = zero16();
#pragma unroll
  for (int q = 0; q < G::KD; ++q) E::mma(Wt[(l * G::KD + q) * 64 + lane], xf[q], acc);
#pragma unroll
  for (int t = 0; t < G::PE; ++t) pre[l * G::PE + t] = E::NSPLIT == 2 ? acc[t] + acc[t + 8] : acc[t];
}

// dX A operand: W^T[c][e] for the contraction dX = dPre . W.  bf16 entries e
// cover (hp, W_hi, dPre_hi), (hp, W_hi, dPre_lo), (hp, W_lo, dPre_hi).
template <typename T, class G>
__device__ void build_wt_frags(const float* __restrict__ W, int ld, int L, int P,
                               typename Eng<T>::frag* __restrict__ WTf) {
  using E = Eng<T>;
  for (int idx = threadIdx.x; idx < G::CT * G::NQS * 64; idx += blockDim.x) {
    const int lane = idx & 63;
    const int qs = (idx >> 6) % G::NQS;
    const int ct = (idx >> 6) / G::NQS;
    const int c = 32 * ct + (lane & 31), h = lane >> 5;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 16 * qs + 8 * h + i;
      float w = 0.f;
      if (e < G::NE) {
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
    WTf[idx] = E::pack(v);
  }
}

__device__ __forceinline__ void wave_lds_sync();

// ---------------------------------------------------------------- per-token front end
// Branch-free load of a token row's projection B operand.  Callers clamp the
// row to a valid one and discard or zero the features of tokens past the end,
// so prefetched loads never sit behind a data-dependent branch (which would
// make the compiler wait for them early).
template <typename T, class G>
__device__ __forceinline__ void load_row_frags_nb(const T* __restrict__ x, typename Eng<T>::frag (&xf)[G::KD]) {
  using E = Eng<T>;
  const int h = lane_id() >> 5;
#pragma unroll
  for (int q = 0; q < G::KD; ++q) xf[q] = *reinterpret_cast<const typename E::frag*>(x + 16 * q + 8 * h);
}

// Load the B operand of the projection for token row `x` (nullptr -> zeros).
template <typename T, class G>
__device__ __forceinline__ void load_row_frags(const T* __restrict__ x, typename Eng<T>::frag (&xf)[G::KD]) {
  using E = Eng<T>;
  const int h = lane_id() >> 5;
  if (x) {
#pragma unroll
    for (int q = 0; q < G::KD; ++q) xf[q] = *reinterpret_cast<const typename E::frag*>(x + 16 * q + 8 * h);
  } else {
#pragma unroll
    for (int q = 0; q < G::KD; ++q) xf[q] = E::zero();
  }
}

// float32 I/O: pre[hp] = W_hp . x for slots [HP0, HP1) from the plain rows
// Wr (build_proj_frags), accumulated in float64 and rounded once.  In float32
// the partial sums of a d-term dot product grow to about sqrt(d) |w| |x|, so
// their rounding leaves an absolute error of ~1e-6 on pre at d = 128, which
// beta carries into the logits; in float64 only the final rounding remains.
// Each lane half sums its 8 KD columns of the token, then the halves are added.
template <class G, int HP0, int HP1>
__device__ __forceinline__ void project_rows_f64(const float* __restrict__ Wr, const f32x8 (&xf)[G::KD],
                                                 float (&pre)[G::NHP]) {
  const int h = lane_id() >> 5;
  constexpr int NH = HP1 > HP0 ? HP1 - HP0 : 1;
  double s[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) s[j] = 0.0;
  // columns outer, one float64 sum per hyperplane: only the current step's
  // row pieces are live
#pragma unroll
  for (int q = 0; q < G::KD; ++q) {
#pragma unroll
    for (int j = 0; j < HP1 - HP0; ++j) {
      const f32x8 w = *reinterpret_cast<const f32x8*>(Wr + (HP0 + j) * G::D + 16 * q + 8 * h);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[j] = fma((double)w[i], (double)xf[q][i], s[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int hp = 0; hp < G::NHP; ++hp) pre[hp] = 0.f;
#pragma unroll
  for (int j = 0; j < HP1 - HP0; ++j) pre[HP0 + j] = (float)(s[j] + __shfl_xor(s[j], 32, 64));
}

// Projection tiles [PT0, PT1) that hold the hyperplanes of the tables
// overlapping bucket rows [R0, R0 + NROWS).
template <class G, int R0, int NROWS>
struct WinTiles {
  static constexpr int L0 = R0 / G::R;
  static constexpr int L1 = cdiv(R0 + NROWS, G::R) < G::LMAX ? cdiv(R0 + NROWS, G::R) : G::LMAX;
  static constexpr int PT0 = L1 > L0 ? L0 * G::PE / G::HPT : 0;
  static constexpr int PT1 = L1 > L0 ? cdiv(L1 * G::PE, G::HPT) : 0;
};

// pre[hp] = W_hp . x for the hyperplane slots of projection tiles [PT0, PT1)
// of the lane's token; other slots are 0.
template <typename T, class G, int PT0, int PT1>
__device__ __forceinline__ void project_tiles(const typename Eng<T>::frag* __restrict__ Wf,
                                              const typename Eng<T>::frag (&xf)[G::KD],
                                              float (&pre)[G::NHP]) {
  using E = Eng<T>;
  if constexpr (std::is_same<T, float>::value) {
    project_rows_f64<G, E::HPT * PT0, (E::HPT * PT1 < G::NHP ? E::HPT * PT1 : G::NHP)>(
        reinterpret_cast<const float*>(Wf), xf, pre);
    return;
  }
  const int lane = lane_id();
#pragma unroll
  for (int hp = 0; hp < G::NHP; ++hp) pre[hp] = 0.f;
#pragma unroll
  for (int pt = PT0; pt < PT1; ++pt) {
    f32x16 acc = zero16();
#pragma unroll
    for (int q = 0; q < G::KD; ++q) E::mma(Wf[(pt * G::KD + q) * 64 + lane], xf[q], acc);
    if (E::NSPLIT == 2) {
#pragma unroll
      for (int v = 0; v < 8; ++v)
        if (8 * pt + v < G::NHP) pre[8 * pt + v] = acc[v] + acc[v + 8];
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (16 * pt + v < G::NHP) pre[16 * pt + v] = acc[v];
    }
  }
}

// pre[hp] = W_hp . x for every hyperplane slot of the lane's token.
template <typename T, class G>
__device__ __forceinline__ void project(const typename Eng<T>::frag* __restrict__ Wf,
                                        const typename Eng<T>::frag (&xf)[G::KD],
                                        float (&pre)[G::NHP]) {
  using E = Eng<T>;
  if constexpr (std::is_same<T, float>::value) {
    project_rows_f64<G, 0, G::NHP>(reinterpret_cast<const float*>(Wf), xf, pre);
    return;
  }
  const int lane = lane_id();
#pragma unroll
  for (int pt = 0; pt < G::NPT; ++pt) {
    f32x16 acc = zero16();
#pragma unroll
    for (int q = 0; q < G::KD; ++q) E::mma(Wf[(pt * G::KD + q) * 64 + lane], xf[q], acc);
    if (E::NSPLIT == 2) {
#pragma unroll
      for (int v = 0; v < 8; ++v)
        if (8 * pt + v < G::NHP) pre[8 * pt + v] = acc[v] + acc[v + 8];
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (16 * pt + v < G::NHP) pre[16 * pt + v] = acc[v];
    }
  }
}

// Soft corner assignments in TLAYOUT (slides frame "Soft corner assignments
// make hashing differentiable"; product-of-sigmoids form, reading notes
// section 2.4): phi_r = prod_t sigma(2 beta u_t v_{r,t}), u = tanh(pre).
// Lane half h owns the corners whose bit 2 equals h.  Only bucket rows
// [R0, R0 + NROWS) are produced (R0 and NROWS multiples of 32); rows of tables
// >= L and padding rows are 0.
//
// Both lane halves hold the same token, so of each pair of hyperplanes
// (t, t + 1) half h evaluates tanh and the sigmoid pair of t + h only, and one
// half swap hands every lane both (an odd last hyperplane is evaluated in
// both halves).  ev receives E[v_t] = sigma(2 beta u_t) - sigma(-2 beta u_t)
// = tanh(beta u_t) of the hyperplane this half evaluated, in slot l * PE + t
// of the pair's first hyperplane t (the softmax backward of split tables
// uses it).  BITSEL: each half takes its hyperplane's value with a bit mask
// instead of a select (same value; pre-activations that were loaded rather
// than projected otherwise become one load at a lane-dependent index, which
// moves them out of registers).
template <class G, int R0, int NROWS, bool BITSEL = false>
__device__ __forceinline__ void soft_assign_rows(const float (&pre)[G::NHP], float beta2, int L,
                                                 float (&ev)[G::NHP], float (&phi)[NROWS / 2], bool keep = true,
                                                 float scale = 1.f) {
  static_assert(R0 % 32 == 0 && NROWS % 32 == 0 && R0 + NROWS <= G::LRP, "row window");
  const int h = lane_id() >> 5;
  constexpr int L0 = R0 / G::R;
  constexpr int L1 = cdiv(R0 + NROWS, G::R) < G::LMAX ? cdiv(R0 + NROWS, G::R) : G::LMAX;
#pragma unroll
  for (int l = L0; l < L1; ++l) {
    float sp[G::PE], sm[G::PE];
#pragma unroll
    for (int t = 0; t < G::PE; t += 2) {
      if (t + 1 < G::PE) {
        float x;
        if constexpr (BITSEL) {
          const int m = h ? -1 : 0;
          x = __int_as_float((__float_as_int(pre[l * G::PE + t + 1]) & m) | (__float_as_int(pre[l * G::PE + t]) & ~m));
        } else {
          x = h ? pre[l * G::PE + t + 1] : pre[l * G::PE + t];
        }
        float p, q;
        sigmoid_pair(beta2 * tanh_f(x), p, q);
        ev[l * G::PE + t] = p - q;
        const HalfPair hp = halves(p), hq = halves(q);
        sp[t] = hp.lo; sp[t + 1] = hp.hi;
        sm[t] = hq.lo; sm[t + 1] = hq.hi;
      } else {
        sigmoid_pair(beta2 * tanh_f(pre[l * G::PE + t]), sp[t], sm[t]);
        ev[l * G::PE + t] = sp[t] - sm[t];
      }
    }
    // tables >= L (and every table of a token with keep false) get zero rows,
    // and every row is multiplied by scale: the factor of bit 2 carries both
    // (sigmoids are finite, so the products are exactly 0)
    const float f2 = (l < L && keep) ? (h ? sp[2] : sm[2]) * scale : 0.f;
    float g[4];
    g[0] = sm[0] * sm[1] * f2;
    g[1] = sp[0] * sm[1] * f2;
    g[2] = sm[0] * sp[1] * f2;
    g[3] = sp[0] * sp[1] * f2;
    constexpr int NH = 1 << (G::PE - 3);
    float hi[NH];
    hi[0] = 1.f;
#pragma unroll
    for (int t = 3; t < G::PE; ++t) {
      const int half = 1 << (t - 3);
#pragma unroll
      for (int x = 0; x < half; ++x) {
        hi[x + half] = hi[x] * sp[t];
        hi[x] = hi[x] * sm[t];
      }
    }
#pragma unroll
    for (int a = 0; a < NROWS / 32; ++a) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr0 = R0 + 32 * a + 8 * (v >> 2) + (v & 3);
        if (lr0 / G::R == l) {
          const int r0 = lr0 % G::R;
          phi[16 * a + v] = g[r0 & 3] * hi[r0 >> 3];
        }
      }
    }
  }
#pragma unroll
  for (int a = 0; a < NROWS / 32; ++a)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if ((R0 + 32 * a + 8 * (v >> 2) + (v & 3)) / G::R >= G::LMAX) phi[16 * a + v] = 0.f;
}

template <class G>
__device__ __forceinline__ void soft_assign(const float (&pre)[G::NHP], float beta2, int L,
                                            float (&ev)[G::NHP], float (&phi)[G::LRP / 2]) {
  soft_assign_rows<G, 0, G::LRP>(pre, beta2, L, ev, phi);
}

// B operand of K16 step q from a TLAYOUT vector held in registers.
template <typename T, int M>
__device__ __forceinline__ typename Eng<T>::frag tl_frag(const float (&x)[M / 2], int q) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = x[8 * q + i];
  return Eng<T>::pack(v);
}

template <typename T, int M>
__device__ __forceinline__ void tl_frag_split(const float (&x)[M / 2], int q,
                                              typename Eng<T>::frag& hi, typename Eng<T>::frag& lo) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = x[8 * q + i];
  Eng<T>::split(v, hi, lo);
}

// Backward through softmax, beta, corners and tanh for one token (TLAYOUT).
// dLambda = phi * (dphi - sum_r phi dphi) per table; dU_t = beta sum_r dLambda_r v_{r,t};
// dPre = dU * (1 - u^2) with u = tanh(pre), the derivative taken from pre
// (tanh_sech2).  Both lane halves end with every dPre value.  Works on
// bucket rows [R0, R0 + NROWS), which must hold whole tables; dPre slots of
// tables outside the window are left untouched.  bterm receives the token's
// share of dL/dbeta over these tables: sum_r dLambda_r (u . v_r)
// = sum_t u_t sum_r dLambda_r v_{r,t} (the logits are beta u . v_r).
template <class G, int R0, int NROWS>
__device__ __forceinline__ void assign_backward_rows(const float (&phi)[NROWS / 2], const float (&dphi)[NROWS / 2],
                                                     const float (&pre)[G::NHP], float beta,
                                                     float (&dpre)[G::NHP], float& bterm) {
  const int h = lane_id() >> 5;
  const float sgn2 = h ? 1.f : -1.f;
  constexpr int L0 = R0 / G::R;
  constexpr int L1 = cdiv(R0 + NROWS, G::R) < G::LMAX ? cdiv(R0 + NROWS, G::R) : G::LMAX;
#pragma unroll
  for (int l = L0; l < L1; ++l) {
    float s = 0.f;
#pragma unroll
    for (int a = 0; a < NROWS / 32; ++a)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr0 = R0 + 32 * a + 8 * (v >> 2) + (v & 3);
        if (lr0 / G::R == l) s += phi[16 * a + v] * dphi[16 * a + v];
      }
    s += xor32(s);
    float du[G::PE];
#pragma unroll
    for (int t = 0; t < G::PE; ++t) du[t] = 0.f;
#pragma unroll
    for (int a = 0; a < NROWS / 32; ++a)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr0 = R0 + 32 * a + 8 * (v >> 2) + (v & 3);
        if (lr0 / G::R == l) {
          const int r0 = lr0 % G::R;
          const float dl = phi[16 * a + v] * (dphi[16 * a + v] - s);
#pragma unroll
          for (int t = 0; t < G::PE; ++t) {
            if (t == 2) du[t] += sgn2 * dl;
            else du[t] += ((r0 >> t) & 1) ? dl : -dl;
          }
        }
      }
#pragma unroll
    for (int t = 0; t < G::PE; ++t) {
      const float d = du[t] + xor32(du[t]);
      float uu, s2;
      tanh_sech2(pre[l * G::PE + t], uu, s2);
      dpre[l * G::PE + t] = beta * d * s2;
      bterm += uu * d;
    }
  }
}

// Softmax-backward sums of one token over the 32 corners of a table part
// (bucket rows [R0, R0 + 32), R0 a multiple of 32, 2^PE >= 64): out[0] =
// sum_r phi_r dphi_r and out[1 + t] = sum_r phi_r dphi_r v_{r,t}.  Both lane
// halves end with the sums over the 32 corners.  The parts of a table give
// dU_t = A_t - s E[v_t] with s, A the sums over the whole table and
// E[v_t] = sum_r phi_r v_{r,t} = tanh(beta u_t) (phi factorises over the
// corner bits, each bit a two-way softmax).
template <class G, int R0>
__device__ __forceinline__ void assign_partials_split(const float (&phi)[16], const float (&dphi)[16],
                                                      float (&out)[1 + G::PE]) {
  static_assert(R0 % 32 == 0 && G::R >= 64, "tables of at least 64 corners, 32 per part");
  const int h = lane_id() >> 5;
  // register v holds corner r = R0 % R + 8 (v / 4) + 4 h + v % 4: bits 0, 1
  // of r are bits 0, 1 of v, bits 3, 4 of r bits 2, 3 of v, bit 2 is h and
  // bits 5 and up are fixed per part.  Signed sums over one bit at a time by
  // a butterfly over the bits of v.
  float a[8], m0 = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float lo = phi[2 * j] * dphi[2 * j], hi = phi[2 * j + 1] * dphi[2 * j + 1];
    a[j] = lo + hi;
    m0 += hi - lo;                       // bit 0 of v set: +, clear: -
  }
  float b[4], m1 = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    b[j] = a[2 * j] + a[2 * j + 1];
    m1 += a[2 * j + 1] - a[2 * j];       // bit 1 of v
  }
  const float c0 = b[0] + b[1], c1 = b[2] + b[3];
  const float m2 = (b[1] - b[0]) + (b[3] - b[2]);   // bit 2 of v
  const float sum = c0 + c1, m3 = c1 - c0;          // bit 3 of v
  out[0] = sum;
#pragma unroll
  for (int t = 0; t < G::PE; ++t) {
    float v;
    if (t == 0) v = m0;
    else if (t == 1) v = m1;
    else if (t == 2) v = h ? sum : -sum;
    else if (t == 3) v = m2;
    else if (t == 4) v = m3;
    else v = ((R0 % G::R) >> t) & 1 ? sum : -sum;
    out[1 + t] = v;
  }
#pragma unroll
  for (int i = 0; i <= G::PE; ++i) out[i] += xor32(out[i]);
}

// One token's dPre slots to row[0, NHP): the two lanes that hold the token
// (lane halves h = 0, 1, both with every slot) write one half each.
template <class G>
__device__ __forceinline__ void store_dpre_half(float* __restrict__ row, const float (&dpre)[G::NHP], int h) {
  constexpr int HALF = cdiv(G::NHP, 2);
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const float v = h ? dpre[HALF + i < G::NHP ? HALF + i : G::NHP - 1] : dpre[i];
    if (HALF * h + i < G::NHP) row[HALF * h + i] = v;
  }
}

template <class G, int R0, int NROWS>
__device__ __forceinline__ void assign_backward_rows(const float (&phi)[NROWS / 2], const float (&dphi)[NROWS / 2],
                                                     const float (&pre)[G::NHP], float beta,
                                                     float (&dpre)[G::NHP]) {
  float unused = 0.f;
  assign_backward_rows<G, R0, NROWS>(phi, dphi, pre, beta, dpre, unused);
}

// Sum over the 64 lanes of a wave (every lane ends with the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <class G>
__device__ __forceinline__ void assign_backward(const float (&phi)[G::LRP / 2], const float (&dphi)[G::LRP / 2],
                                                const float (&pre)[G::NHP], float beta, float (&dpre)[G::NHP],
                                                float& bterm) {
  assign_backward_rows<G, 0, G::LRP>(phi, dphi, pre, beta, dpre, bterm);
}

// MFMA operand (bf16) with k over 16 consecutive rows of a row-major LDS tile
// and one column per lane: lane (n, h) receives M[r0 + kmap(0, h, i)][col0 + n]
// for i = 0..7.  Two transposing LDS loads (ds_read_b64_tr_b16): within each
// group of 16 lanes, lane 4a + b receives element b of the 8-byte pieces that
// lanes a, a + 4, a + 8 and a + 12 address (measured on gfx950).  So lane L
// addresses row r0 + 4 (L / 32) + (L / 4) % 4 (+ 8 for the second load) at
// the run of 4 columns col0 + 16 ((L / 16) % 2) + 4 (L % 4); pos(c) is the
// storage position of the run that starts at column c (c a multiple of 4).
typedef short i16x4 __attribute__((ext_vector_type(4)));
template <class Pos>
__device__ __forceinline__ bf16x8 load_kcol_tr(const bf16* tile, int stride, int r0, int col0, Pos pos) {
  const int L = lane_id();
  const int row = r0 + 4 * (L >> 5) + ((L >> 2) & 3);
  const int col = col0 + 16 * ((L >> 4) & 1) + 4 * (L & 3);
  const bf16* p0 = tile + row * stride + pos(col);
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 8 * stride));
  // whole-vector reinterpretation (per-element casts were packed wrongly)
  const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
  return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Storage position of a run of 4 columns starting at c in a row kept in kmap
// frag order (column 16 q + 8 hh + e at 16 q + 8 (e / 4) + 4 hh + e % 4):
// runs 0, 1, 2, 3 of a 16-column group sit at runs 0, 2, 1, 3.
__device__ __forceinline__ int kmap_run_pos(int c) {
  const int r = (c >> 2) & 3;
  return (c & ~15) + 4 * (((r & 1) << 1) | (r >> 1));
}

// Order this wave's LDS writes before its later LDS reads of other lanes'
// data (a wave issues LDS instructions in order; this stops the compiler
// from moving them and waits for the writes to land).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// B operand of the dX contraction, step qs (entries e = 16 qs + 8 h + i).
template <typename T, class G>
__device__ __forceinline__ typename Eng<T>::frag dpre_frag(const float (&dpre)[G::NHP], int qs) {
  using E = Eng<T>;
  const int h = lane_id() >> 5;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float a = 0.f, b = 0.f;   // values for h = 0 and h = 1
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int e = 16 * qs + 8 * hh + i;
      float w = 0.f;
      if (e < G::NE) {
        const int hp = e % G::NHP, which = e / G::NHP;
        const float x = dpre[hp];
        if (E::NSPLIT == 2) {
          const float xh = E::round(x);
          w = (which == 1) ? (x - xh) : xh;
        } else {
          w = x;
        }
      }
      if (hh == 0) a = w; else b = w;
    }
    v[i] = h ? b : a;
  }
  return E::pack(v);
}

// Store a TLAYOUT row of D values (4 consecutive columns per register group).
template <typename T, int D>
__device__ __forceinline__ void store_tl_row(T* __restrict__ row, const float (&x)[D / 2]) {
  const int h = lane_id() >> 5;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      typename Eng<T>::vec4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = (T)x[16 * mt + 4 * j + k];
      *reinterpret_cast<typename Eng<T>::vec4*>(row + 32 * mt + 8 * j + 4 * h) = w;
    }
}

// Store one 32-column tile (accumulator of a C^T[c][tok] MFMA) of a token row.
template <typename T>
__device__ __forceinline__ void store_tl_tile(T* __restrict__ row, int ct, const f32x16& acc, float scale) {
  const int h = lane_id() >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    typename Eng<T>::vec4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = (T)(acc[4 * j + k] * scale);
    *reinterpret_cast<typename Eng<T>::vec4*>(row + 32 * ct + 8 * j + 4 * h) = w;
  }
}

// Output staging: a wave writes its 32 x D output tile into LDS (row stride
// D + 8 elements) from TLAYOUT accumulators, then stores whole rows with
// 16-byte lanes (four 256-byte rows per instruction at d = 128).
template <int D, typename T>
struct OutStage {
  static constexpr int SP = D + 8;
  static constexpr int ELEMS = 32 * SP;
  __device__ __forceinline__ static void put(T* __restrict__ st, int ct, const f32x16& acc, float scale) {
    const int lane = lane_id(), n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      typename Eng<T>::vec4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = (T)(acc[4 * j + k] * scale);
      *reinterpret_cast<typename Eng<T>::vec4*>(st + n * SP + 32 * ct + 8 * j + 4 * h) = w;
    }
  }
  // rows t0 .. t0+31 of out (only rows < t_end are written)
  __device__ __forceinline__ static void flush(const T* __restrict__ st, T* __restrict__ out, int64_t t0,
                                               int64_t t_end) {
    constexpr int EPC = 16 / (int)sizeof(T);
    constexpr int CPR = D / EPC;
    const int lane = lane_id();
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < 32 * CPR / 64; ++it) {
      const int flat = it * 64 + lane;
      const int row = flat / CPR, ch = flat % CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(st + row * SP + ch * EPC);
      if (t0 + row < t_end) *reinterpret_cast<uint4*>(out + (t0 + row) * D + ch * EPC) = v;
    }
    wave_lds_sync();
  }
};

template <typename T, int D>
__device__ __forceinline__ void load_tl_row(const T* __restrict__ row, float (&x)[D / 2]) {
  const int h = lane_id() >> 5;
#pragma unroll
  for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      typename Eng<T>::vec4 w = *reinterpret_cast<const typename Eng<T>::vec4*>(row + 32 * mt + 8 * j + 4 * h);
#pragma unroll
      for (int k = 0; k < 4; ++k) x[16 * mt + 4 * j + k] = (float)w[k];
    }
}

}  // namespace race
