// Non-causal RACE attention kernels for gfx950.
//
//   race_bucket_reduce  content^(l) = Phi_K^(l)^T V, mass^(l) = Phi_K^(l)^T 1
//                       (slides frame "Each bucket stores mass and a weighted
//                       value sum"): per-workgroup partial banks, then a
//                       fixed-order sum over workgroups (deterministic).
//   race_readout_norm   O = sum_l Phi_Q content / sum_l Phi_Q mass (slides
//                       frame "Normalize after combining the tables").
//   race_bwd_q          recompute O; g = dO/Den, h = -(dO.O)/Den;
//                       dPhi_Q = content g + mass h -> dQ; reduce
//                       dcontent = Phi_Q^T g, dmass = Phi_Q^T h.
//   race_bwd_kv         dV = sum_l Phi_K dcontent; dPhi_K = dcontent V + dmass -> dK.
//
// Every kernel fuses the soft bucketing of its token rows (projection on
// MFMA, tanh and sigmoids on VALU); Phi never reaches HBM.  Bucket banks are
// float32.  With bf16 I/O the float32 operands of each contraction (bucket
// bank, projection rows, gradients that may cancel) are split into bf16
// hi + lo parts; per-token soft assignments are rounded to bf16 once and the
// same rounded values feed both numerator and denominator.
#pragma once
#include "race_device.hpp"

namespace race {

struct NCArgs {
  const void* X;            // Q (readout, bwd_q) or K (reduce, bwd_kv)
  const void* Y;            // V (reduce, bwd_kv) or dO (bwd_q)
  void* out0;               // O (readout), dQ (bwd_q), dV (bwd_kv)
  void* out1;               // dK (bwd_kv)
  Tables W;
  const float* st_content;  // [BH][LRP][d]   bucket (or gradient) bank
  const float* st_mass;     // [BH][LRP]
  float* part;              // [BH][nchunk][LRP][d+1] partial banks
  float beta;
  int L, P;
  int64_t N;
  int64_t chunk_tokens;     // tokens per workgroup
  int nchunk;
  // backward kernels: when set, each wave writes its share of dL/dbeta to
  // dbeta_part[(bh * nchunk + chunk) * 4 + wave]
  float* dbeta_part;
  // backward kernels: when set, dL/dPre of every token, float32 [BH][N][NHP]
  // (hyperplane slot l * PE + t), for the table gradient
  float* dpre_out;
};

constexpr int TT = 128;     // tokens per workgroup iteration (4 waves x 32)

// Token tiles of one workgroup of the non-causal kernels.  Interleaved: the
// grid sweeps each tensor front to back together, one tile per workgroup per
// sweep (workgroup slot c takes tiles c, c + nchunk, c + 2 nchunk, ...), so
// neighbouring workgroups read neighbouring rows.  Workgroups are dealt to
// the 8 XCDs round-robin by linear id; with nchunk a multiple of 8 the slots
// are ordered so that each XCD's workgroups take one contiguous eighth of
// every sweep.  Contiguous: one run of chunk_tokens tokens per workgroup.
// Either way every tile is taken by one workgroup and the partial banks are
// summed in workgroup order.
constexpr bool kInterleaveTiles = true;
struct TileSpan {
  int64_t begin, end, step;   // first tile's first token, token bound, stride between tiles
};
__device__ __forceinline__ TileSpan tile_span(const NCArgs& a, int chunk) {
  if (kInterleaveTiles) {
    int64_t c = chunk;
    if (a.nchunk % 8 == 0) c = (int64_t)(chunk % 8) * (a.nchunk / 8) + chunk / 8;
    return {c * TT, a.N, (int64_t)a.nchunk * TT};
  }
  const int64_t b = (int64_t)chunk * a.chunk_tokens;
  return {b, min(a.N, b + a.chunk_tokens), (int64_t)TT};
}

// Row padding (elements) of LDS staging tiles: keeps 16-byte (bf16) and
// 32-byte (float32) fragment rows aligned and shifts rows across banks.
template <typename T> struct Pad { static constexpr int v = 8; };

// A operand of the readout: rows = value columns c (CT tiles) plus one tile
// whose every row is the mass, so the denominator comes out of the same MFMA
// with the same rounded Phi_Q.  k over buckets follows kmap.
template <typename T, class G>
__device__ void build_readout_frags(const float* __restrict__ content, const float* __restrict__ mass,
                                    typename Eng<T>::frag* __restrict__ RF) {
  using E = Eng<T>;
  constexpr int NS = E::NSPLIT;
  for (int idx = threadIdx.x; idx < (G::CT + 1) * G::KL * NS * 64; idx += blockDim.x) {
    const int lane = idx & 63;
    const int sp = (idx >> 6) % NS;
    const int q = ((idx >> 6) / NS) % G::KL;
    const int mt = ((idx >> 6) / NS) / G::KL;
    const int c = 32 * mt + (lane & 31), h = lane >> 5;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int lr = kmap(q, h, i);
      v[i] = (mt < G::CT) ? content[(size_t)lr * G::D + c] : mass[lr];
    }
    typename E::frag hi, lo;
    E::split(v, hi, lo);
    RF[idx] = sp ? lo : hi;
  }
}

// A operand bank[lr][c] with rows = buckets and k over columns c, either by
// kmap (B operand from a TLAYOUT register vector) or by the plain row map
// c = 16 q + 8 h + i (B operand loaded straight from a token row).
template <typename T, class G, bool KMAP>
__device__ void build_bank_rows_frags(const float* __restrict__ content, typename Eng<T>::frag* __restrict__ DF) {
  using E = Eng<T>;
  constexpr int NS = E::NSPLIT;
  for (int idx = threadIdx.x; idx < G::AT * G::KD * NS * 64; idx += blockDim.x) {
    const int lane = idx & 63;
    const int sp = (idx >> 6) % NS;
    const int q = ((idx >> 6) / NS) % G::KD;
    const int at = ((idx >> 6) / NS) / G::KD;
    const int lr = 32 * at + (lane & 31), h = lane >> 5;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = KMAP ? kmap(q, h, i) : 16 * q + 8 * h + i;
      v[i] = content[(size_t)lr * G::D + c];
    }
    typename E::frag hi, lo;
    E::split(v, hi, lo);
    DF[idx] = sp ? lo : hi;
  }
}

// A operand bank^T[c][lr] (rows = columns c, k over buckets by kmap), no mass tile.
template <typename T, class G>
__device__ void build_bank_cols_frags(const float* __restrict__ content, typename Eng<T>::frag* __restrict__ VF) {
  using E = Eng<T>;
  constexpr int NS = E::NSPLIT;
  for (int idx = threadIdx.x; idx < G::CT * G::KL * NS * 64; idx += blockDim.x) {
    const int lane = idx & 63;
    const int sp = (idx >> 6) % NS;
    const int q = ((idx >> 6) / NS) % G::KL;
    const int mt = ((idx >> 6) / NS) / G::KL;
    const int c = 32 * mt + (lane & 31), h = lane >> 5;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = content[(size_t)kmap(q, h, i) * G::D + c];
    typename E::frag hi, lo;
    E::split(v, hi, lo);
    VF[idx] = sp ? lo : hi;
  }
}

// Readout of one token (TLAYOUT): acc[mt] = bank^T[mt] . Phi^T, acc[CT] = Den.
template <typename T, class G>
__device__ __forceinline__ void readout_mma(const typename Eng<T>::frag* __restrict__ RF,
                                            const float (&phi)[G::LRP / 2], f32x16 (&acc)[G::CT + 1]) {
  using E = Eng<T>;
  constexpr int NS = E::NSPLIT;
  const int lane = lane_id();
#pragma unroll
  for (int mt = 0; mt <= G::CT; ++mt) acc[mt] = zero16();
#pragma unroll
  for (int q = 0; q < G::KL; ++q) {
    const typename E::frag b = tl_frag<T, G::LRP>(phi, q);
#pragma unroll
    for (int mt = 0; mt <= G::CT; ++mt)
#pragma unroll
      for (int sp = 0; sp < NS; ++sp) E::mma(RF[((mt * G::KL + q) * NS + sp) * 64 + lane], b, acc[mt]);
  }
}

// dX = dPre . W for one token (TLAYOUT over columns).
template <typename T, class G>
__device__ __forceinline__ void dx_mma(const typename Eng<T>::frag* __restrict__ WTf,
                                       const float (&dpre)[G::NHP], float (&dx)[G::D / 2]) {
  using E = Eng<T>;
  const int lane = lane_id();
  typename E::frag bq[G::NQS];
#pragma unroll
  for (int qs = 0; qs < G::NQS; ++qs) bq[qs] = dpre_frag<T, G>(dpre, qs);
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) {
    f32x16 acc = zero16();
#pragma unroll
    for (int qs = 0; qs < G::NQS; ++qs) E::mma(WTf[(ct * G::NQS + qs) * 64 + lane], bq[qs], acc);
#pragma unroll
    for (int v = 0; v < 16; ++v) dx[16 * ct + v] = acc[v];
  }
}

// dX = dPre . W for the wave's 32 tokens, written into the staging tile.
template <typename T, class G>
__device__ __forceinline__ void dx_mma_stage(const typename Eng<T>::frag* __restrict__ WTf,
                                             const float (&dpre)[G::NHP], T* __restrict__ st) {
  using E = Eng<T>;
  const int lane = lane_id();
  typename E::frag bq[G::NQS];
#pragma unroll
  for (int qs = 0; qs < G::NQS; ++qs) bq[qs] = dpre_frag<T, G>(dpre, qs);
#pragma unroll
  for (int ct = 0; ct < G::CT; ++ct) {
    f32x16 acc = zero16();
#pragma unroll
    for (int qs = 0; qs < G::NQS; ++qs) E::mma(WTf[(ct * G::NQS + qs) * 64 + lane], bq[qs], acc);
    OutStage<G::D, T>::put(st, ct, acc, 1.f);
  }
}

// Cooperative bucket reduction of one 128-token tile: acc[j] (tile w + 4 j of
// the (AT) x (CT + 1) grid) += PhiT[lr][tok] * [B | extra][tok][c].
// The extra column tile is all ones (mass) or hs[tok] (gradient mass).
template <typename T, class G, int TTP, int BSP, int NTW>
__device__ __forceinline__ void reduce_tile_mma(const T* __restrict__ PhiT, const T* __restrict__ Bs,
                                                const float* __restrict__ hs, f32x16 (&acc)[NTW]) {
  using E = Eng<T>;
  constexpr int NTILE = G::AT * (G::CT + 1);
  const int lane = lane_id(), n = lane & 31, h = lane >> 5, w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int tidx = w + 4 * j;
    if (tidx < NTILE) {
      const int at = tidx / (G::CT + 1), ct = tidx % (G::CT + 1);
#pragma unroll
      for (int s = 0; s < TT / 16; ++s) {
        const typename E::frag af =
            *reinterpret_cast<const typename E::frag*>(PhiT + (32 * at + n) * TTP + 16 * s + 8 * h);
        typename E::frag bf;
        if (ct < G::CT) {
#pragma unroll
          for (int i = 0; i < 8; ++i) bf[i] = Bs[(16 * s + 8 * h + i) * BSP + 32 * ct + n];
        } else if (hs) {
#pragma unroll
          for (int i = 0; i < 8; ++i) bf[i] = (T)hs[16 * s + 8 * h + i];
        } else {
          bf = E::ones();
        }
        E::mma(af, bf, acc[j]);
      }
    }
  }
}

template <typename T, class G, int NTW>
__device__ __forceinline__ void write_partials(float* __restrict__ part, const f32x16 (&acc)[NTW]) {
  constexpr int NTILE = G::AT * (G::CT + 1);
  const int lane = lane_id(), n = lane & 31, h = lane >> 5, w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int tidx = w + 4 * j;
    if (tidx < NTILE) {
      const int at = tidx / (G::CT + 1), ct = tidx % (G::CT + 1);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = 32 * at + 8 * (v >> 2) + 4 * h + (v & 3);
        if (ct < G::CT) part[(size_t)lr * (G::D + 1) + 32 * ct + n] = acc[j][v];
        else if (n == 0) part[(size_t)lr * (G::D + 1) + G::D] = acc[j][v];
      }
    }
  }
}

// ------------------------------------------------------------------ race_bucket_reduce
template <typename T, class G>
__global__ __launch_bounds__(256) void race_bucket_reduce(NCArgs a) {
  using E = Eng<T>;
  using frag = typename E::frag;
  constexpr int TTP = TT + Pad<T>::v;
  constexpr int BSP = G::D + Pad<T>::v;
  constexpr int NTW = cdiv(G::AT * (G::CT + 1), 4);
  __shared__ frag Wf[G::NPT * G::KD * 64];
  __shared__ T PhiT[G::LRP * TTP];
  __shared__ T Bs[TT * BSP];

  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int lane = lane_id(), n = lane & 31, h = lane >> 5, w = threadIdx.x >> 6;
  build_proj_frags<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, Wf);
  __syncthreads();

  const T* X = static_cast<const T*>(a.X) + (size_t)bh * a.N * G::D;
  const T* Y = static_cast<const T*>(a.Y) + (size_t)bh * a.N * G::D;
  const TileSpan span = tile_span(a, chunk);
  const int64_t t_begin = span.begin, t_end = span.end, step = span.step;
  const float beta2 = 2.f * a.beta;

  f32x16 acc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) acc[j] = zero16();

  constexpr int CPR = G::D * (int)sizeof(T) / 16;      // 16-byte chunks per row
  constexpr int NCH = 32 * CPR / 64;                    // chunks per lane per tile
  const int tl = 32 * w + n;
  const int64_t last = t_end - 1;
  // one register set per operand: the next tile's key rows are loaded as
  // soon as this tile's projection has consumed them, its value rows as soon
  // as this tile's are in LDS; both loads stay in flight through the rest of
  // the tile (fewer registers: two waves per SIMD)
  frag xa[G::KD];
  uint4 ya[NCH];
  auto load_x = [&](int64_t b) { load_row_frags_nb<T, G>(X + min(b + tl, last) * G::D, xa); };
  auto load_y = [&](int64_t b) {
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int flat = it * 64 + lane;
      const int row = flat / CPR, ch = flat % CPR;
      const int64_t trow = min(b + 32 * w + row, last);
      ya[it] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(Y + trow * G::D) + 16 * ch);
    }
  };
  load_x(t_begin);
  load_y(t_begin);
  for (int64_t base = t_begin; base < t_end; base += step) {
    const int64_t tok = base + tl;
    const bool valid = tok < t_end;
    float pre[G::NHP], ev[G::NHP], phi[G::LRP / 2];
    project<T, G>(Wf, xa, pre);
    load_x(base + step);
    soft_assign<G>(pre, beta2, a.L, ev, phi);
#pragma unroll
    for (int at = 0; at < G::AT; ++at)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = 32 * at + 8 * (v >> 2) + 4 * h + (v & 3);
        PhiT[lr * TTP + tl] = valid ? (T)phi[16 * at + v] : (T)0.f;
      }
#pragma unroll
    for (int it = 0; it < NCH; ++it) {
      const int flat = it * 64 + lane;
      const int row = flat / CPR, ch = flat % CPR;
      const int64_t trow = base + 32 * w + row;
      const uint4 val = trow < t_end ? ya[it] : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(Bs + (32 * w + row) * BSP) + 16 * ch) = val;
    }
    load_y(base + step);
    __syncthreads();
    reduce_tile_mma<T, G, TTP, BSP, NTW>(PhiT, Bs, nullptr, acc);
    __syncthreads();
  }
  write_partials<T, G, NTW>(a.part + ((size_t)bh * a.nchunk + chunk) * G::LRP * (G::D + 1), acc);
}

// ------------------------------------------------------------------ race_readout_norm
template <typename T, class G>
__global__ __launch_bounds__(256) void race_readout_norm(NCArgs a) {
  using E = Eng<T>;
  using frag = typename E::frag;
  __shared__ frag Wf[G::NPT * G::KD * 64];
  __shared__ frag RF[(G::CT + 1) * G::KL * E::NSPLIT * 64];
  __shared__ T OS[4][OutStage<G::D, T>::ELEMS];
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int lane = lane_id(), n = lane & 31, w = threadIdx.x >> 6;
  build_proj_frags<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, Wf);
  build_readout_frags<T, G>(a.st_content + (size_t)bh * G::LRP * G::D, a.st_mass + (size_t)bh * G::LRP, RF);
  __syncthreads();

  const T* X = static_cast<const T*>(a.X) + (size_t)bh * a.N * G::D;
  T* O = static_cast<T*>(a.out0) + (size_t)bh * a.N * G::D;
  const TileSpan span = tile_span(a, chunk);
  const int64_t t_begin = span.begin, t_end = span.end, step = span.step;
  const float beta2 = 2.f * a.beta;

  const int64_t last = t_end - 1;
  // one 32-token tile: rows in cx (loaded one tile ahead)
  auto tile = [&](const frag (&cx)[G::KD], int64_t base) {
    const int64_t tok = base + n;
    const bool valid = tok < t_end;
    float pre[G::NHP], ev[G::NHP], phi[G::LRP / 2];
    project<T, G>(Wf, cx, pre);
    soft_assign<G>(pre, beta2, a.L, ev, phi);
    f32x16 acc[G::CT + 1];
    readout_mma<T, G>(RF, phi, acc);
    const float inv = 1.f / acc[G::CT][0];
    (void)valid;
#pragma unroll
    for (int mt = 0; mt < G::CT; ++mt) OutStage<G::D, T>::put(OS[w], mt, acc[mt], inv);
    OutStage<G::D, T>::flush(OS[w], O, base, t_end);
  };
  // double-buffered rows: each half prefetches into the set the other half uses
  frag xa[G::KD], xb[G::KD];
  int64_t base = t_begin + 32 * w;
  load_row_frags_nb<T, G>(X + min(base + n, last) * G::D, xa);
  while (base < t_end) {
    load_row_frags_nb<T, G>(X + min(base + step + n, last) * G::D, xb);
    __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of this tile's work
    tile(xa, base);
    base += step;
    if (base >= t_end) break;
    load_row_frags_nb<T, G>(X + min(base + step + n, last) * G::D, xa);
    __builtin_amdgcn_sched_barrier(0);
    tile(xb, base);
    base += step;
  }
}

// ------------------------------------------------------------------ race_bwd_q
// Per token (Den from float32 Phi_Q):
//   A[lr]   = content[lr] . dO          (bank hi + lo times the exact dO row)
//   h       = -(dO . Num) / Den^2 = -(sum_lr phi[lr] A[lr]) / Den^2
//   dPhi_Q  = A / Den + mass h
// and the gradient bank is (Phi_Q / Den)^T dO with mass column -(dO . O).
// Held to two waves per SIMD (at most 256 registers per wave): at one wave
// per SIMD this kernel runs about 10% slower.
template <typename T, class G>
__global__ __launch_bounds__(256, 2) void race_bwd_q(NCArgs a) {
  using E = Eng<T>;
  using frag = typename E::frag;
  constexpr int NS = E::NSPLIT;
  constexpr int TTP = TT + Pad<T>::v;
  constexpr int BSP = G::D + Pad<T>::v;
  constexpr int NTW = cdiv(G::AT * (G::CT + 1), 4);
  __shared__ frag Wf[G::NPT * G::KD * 64];
  __shared__ frag DF[G::AT * G::KD * NS * 64];
  __shared__ frag WTf[G::CT * G::NQS * 64];
  __shared__ float massL[G::LRP];
  __shared__ T PhiT[G::LRP * TTP];
  __shared__ T Bs[TT * BSP];
  __shared__ float hs[TT];
  static_assert(BSP == OutStage<G::D, T>::SP, "dQ is staged in the wave's rows of Bs");

  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int lane = lane_id(), n = lane & 31, h = lane >> 5, w = threadIdx.x >> 6;
  const float* content = a.st_content + (size_t)bh * G::LRP * G::D;
  const float* mass = a.st_mass + (size_t)bh * G::LRP;
  build_proj_frags<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, Wf);
  build_bank_rows_frags<T, G, false>(content, DF);
  build_wt_frags<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, WTf);
  for (int i = threadIdx.x; i < G::LRP; i += blockDim.x) massL[i] = mass[i];
  __syncthreads();

  const T* X = static_cast<const T*>(a.X) + (size_t)bh * a.N * G::D;
  const T* dO = static_cast<const T*>(a.Y) + (size_t)bh * a.N * G::D;
  T* dQ = static_cast<T*>(a.out0) + (size_t)bh * a.N * G::D;
  const TileSpan span = tile_span(a, chunk);
  const int64_t t_begin = span.begin, t_end = span.end, step = span.step;
  const float beta2 = 2.f * a.beta;

  f32x16 racc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) racc[j] = zero16();

  const int tl = 32 * w + n;
  const int64_t last = t_end - 1;
  float bsum = 0.f;
  // one register set per operand: the next tile's Q rows are loaded as soon
  // as this tile's projection has consumed them, its dO rows as soon as this
  // tile's are staged in LDS; both loads stay in flight through the rest of
  // the tile
  frag xa[G::KD], ya[G::KD];
  auto load_x = [&](int64_t b) { load_row_frags_nb<T, G>(X + min(b + tl, last) * G::D, xa); };
  auto load_y = [&](int64_t b) { load_row_frags_nb<T, G>(dO + min(b + tl, last) * G::D, ya); };
  auto tile = [&](int64_t base) {
    const int64_t tok = base + tl;
    const bool valid = tok < t_end;
    frag cy[G::KD];
#pragma unroll
    for (int q = 0; q < G::KD; ++q) cy[q] = valid ? ya[q] : E::zero();
    float pre[G::NHP], ev[G::NHP], phi[G::LRP / 2];
    project<T, G>(Wf, xa, pre);
    load_x(base + step);
    soft_assign<G>(pre, beta2, a.L, ev, phi);
    if (!valid) {
#pragma unroll
      for (int i = 0; i < G::LRP / 2; ++i) phi[i] = 0.f;
    }
    // Den = sum_lr phi mass;  A = content . dO
    float den = 0.f;
#pragma unroll
    for (int at = 0; at < G::AT; ++at)
#pragma unroll
      for (int v = 0; v < 16; ++v) den += phi[16 * at + v] * massL[32 * at + 8 * (v >> 2) + 4 * h + (v & 3)];
    den += xor32(den);
    const float inv = valid ? 1.f / den : 0.f;
    float av[G::LRP / 2];
#pragma unroll
    for (int at = 0; at < G::AT; ++at) {
      f32x16 d = zero16();
#pragma unroll
      for (int q = 0; q < G::KD; ++q)
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) E::mma(DF[((at * G::KD + q) * NS + sp) * 64 + lane], cy[q], d);
#pragma unroll
      for (int v = 0; v < 16; ++v) av[16 * at + v] = d[v];
    }
    float hd = 0.f;
#pragma unroll
    for (int i = 0; i < G::LRP / 2; ++i) hd += phi[i] * av[i];
    hd += xor32(hd);                           // dO . Num
    const float hval = -hd * inv * inv;        // h = -(dO . O) / Den
    float dphi[G::LRP / 2];
#pragma unroll
    for (int at = 0; at < G::AT; ++at)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = 32 * at + 8 * (v >> 2) + 4 * h + (v & 3);
        dphi[16 * at + v] = av[16 * at + v] * inv + massL[lr] * hval;
      }
    float dpre[G::NHP], bterm = 0.f;
    assign_backward<G>(phi, dphi, pre, a.beta, dpre, bterm);
    if (valid && h == 0) bsum += bterm;
    if (a.dpre_out && valid) store_dpre_half<G>(a.dpre_out + ((size_t)bh * a.N + tok) * G::NHP, dpre, h);
    // the wave's 32 rows of Bs are free until the dO rows are staged below
    dx_mma_stage<T, G>(WTf, dpre, Bs + 32 * w * BSP);
    OutStage<G::D, T>::flush(Bs + 32 * w * BSP, dQ, base + 32 * w, t_end);

    // stage (Phi_Q / Den)^T, dO rows and -(dO . O) for the gradient bank
#pragma unroll
    for (int at = 0; at < G::AT; ++at)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = 32 * at + 8 * (v >> 2) + 4 * h + (v & 3);
        PhiT[lr * TTP + tl] = (T)(phi[16 * at + v] * inv);
      }
#pragma unroll
    for (int q = 0; q < G::KD; ++q)
      *reinterpret_cast<frag*>(Bs + tl * BSP + 16 * q + 8 * h) = cy[q];
    load_y(base + step);
    if (h == 0) hs[tl] = valid ? -hd * inv : 0.f;
    __syncthreads();
    reduce_tile_mma<T, G, TTP, BSP, NTW>(PhiT, Bs, hs, racc);
    __syncthreads();
  };
  load_x(t_begin);
  load_y(t_begin);
  for (int64_t base = t_begin; base < t_end; base += step) tile(base);
  write_partials<T, G, NTW>(a.part + ((size_t)bh * a.nchunk + chunk) * G::LRP * (G::D + 1), racc);
  if (a.dbeta_part) {
    bsum = wave_sum(bsum);
    if (lane == 0) a.dbeta_part[((size_t)bh * a.nchunk + chunk) * 4 + w] = bsum;
  }
}

// ------------------------------------------------------------------ race_bwd_kv
template <typename T, class G>
__global__ __launch_bounds__(256) void race_bwd_kv(NCArgs a) {
  using E = Eng<T>;
  using frag = typename E::frag;
  constexpr int NS = E::NSPLIT;
  __shared__ frag Wf[G::NPT * G::KD * 64];
  __shared__ frag VF[G::CT * G::KL * NS * 64];
  __shared__ frag KF[G::AT * G::KD * NS * 64];
  __shared__ frag WTf[G::CT * G::NQS * 64];
  __shared__ float dmassL[G::LRP];
  __shared__ T OS[4][OutStage<G::D, T>::ELEMS];

  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int lane = lane_id(), n = lane & 31, h = lane >> 5, w = threadIdx.x >> 6;
  const float* dcontent = a.st_content + (size_t)bh * G::LRP * G::D;
  const float* dmass = a.st_mass + (size_t)bh * G::LRP;
  build_proj_frags<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, Wf);
  build_bank_cols_frags<T, G>(dcontent, VF);
  build_bank_rows_frags<T, G, false>(dcontent, KF);
  build_wt_frags<T, G>(a.W.at(bh), a.W.ld, a.L, a.P, WTf);
  for (int i = threadIdx.x; i < G::LRP; i += blockDim.x) dmassL[i] = dmass[i];
  __syncthreads();

  const T* Kx = static_cast<const T*>(a.X) + (size_t)bh * a.N * G::D;
  const T* Vx = static_cast<const T*>(a.Y) + (size_t)bh * a.N * G::D;
  T* dV = static_cast<T*>(a.out0) + (size_t)bh * a.N * G::D;
  T* dK = static_cast<T*>(a.out1) + (size_t)bh * a.N * G::D;
  const TileSpan span = tile_span(a, chunk);
  const int64_t t_begin = span.begin, t_end = span.end, step = span.step;
  const float beta2 = 2.f * a.beta;

  const int64_t last = t_end - 1;
  float bsum = 0.f;
  auto tile = [&](const frag (&cx)[G::KD], const frag (&cy)[G::KD], int64_t base) {
    const int64_t tok = base + n;
    const bool valid = tok < t_end;
    float pre[G::NHP], ev[G::NHP], phi[G::LRP / 2];
    project<T, G>(Wf, cx, pre);
    soft_assign<G>(pre, beta2, a.L, ev, phi);
    // dV = sum_l Phi_K dcontent
    frag pb[G::KL];
#pragma unroll
    for (int q = 0; q < G::KL; ++q) pb[q] = tl_frag<T, G::LRP>(phi, q);
#pragma unroll
    for (int ct = 0; ct < G::CT; ++ct) {
      f32x16 acc = zero16();
#pragma unroll
      for (int q = 0; q < G::KL; ++q)
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) E::mma(VF[((ct * G::KL + q) * NS + sp) * 64 + lane], pb[q], acc);
      OutStage<G::D, T>::put(OS[w], ct, acc, 1.f);
    }
    OutStage<G::D, T>::flush(OS[w], dV, base, t_end);
    // dPhi_K[lr] = dcontent[lr] . V + dmass[lr]
    float dphi[G::LRP / 2];
#pragma unroll
    for (int at = 0; at < G::AT; ++at) {
      f32x16 d = zero16();
#pragma unroll
      for (int q = 0; q < G::KD; ++q)
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) E::mma(KF[((at * G::KD + q) * NS + sp) * 64 + lane], cy[q], d);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = 32 * at + 8 * (v >> 2) + 4 * h + (v & 3);
        dphi[16 * at + v] = d[v] + dmassL[lr];
      }
    }
    float dpre[G::NHP], bterm = 0.f;
    assign_backward<G>(phi, dphi, pre, a.beta, dpre, bterm);
    if (valid && h == 0) bsum += bterm;
    if (a.dpre_out && valid) store_dpre_half<G>(a.dpre_out + ((size_t)bh * a.N + tok) * G::NHP, dpre, h);
    dx_mma_stage<T, G>(WTf, dpre, OS[w]);
    OutStage<G::D, T>::flush(OS[w], dK, base, t_end);
  };
  frag xa[G::KD], ya[G::KD], xb[G::KD], yb[G::KD];
  int64_t base = t_begin + 32 * w;
  {
    const int64_t r = min(base + n, last);
    load_row_frags_nb<T, G>(Kx + r * G::D, xa);
    load_row_frags_nb<T, G>(Vx + r * G::D, ya);
  }
  while (base < t_end) {
    {
      const int64_t r = min(base + step + n, last);
      load_row_frags_nb<T, G>(Kx + r * G::D, xb);
      load_row_frags_nb<T, G>(Vx + r * G::D, yb);
    }
    __builtin_amdgcn_sched_barrier(0);
    tile(xa, ya, base);
    base += step;
    if (base >= t_end) break;
    {
      const int64_t r = min(base + step + n, last);
      load_row_frags_nb<T, G>(Kx + r * G::D, xa);
      load_row_frags_nb<T, G>(Vx + r * G::D, ya);
    }
    __builtin_amdgcn_sched_barrier(0);
    tile(xb, yb, base);
    base += step;
  }
  if (a.dbeta_part) {
    bsum = wave_sum(bsum);
    if (lane == 0) a.dbeta_part[((size_t)bh * a.nchunk + chunk) * 4 + w] = bsum;
  }
}

}  // namespace race
