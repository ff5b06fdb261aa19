// Gradient of the projection tables.  The pre-activations of a token row x
// are W^(l) x (slides frame "Soft corner assignments make hashing
// differentiable", paper Algorithm 1), so with dPre the gradient of the loss
// with respect to them,
//   dW^(l)[t][c] = sum over the rows of both sides of dPre[row][l, t] x[row][c]
// (the query rows through Phi_Q, the key rows through Phi_K).  The backward
// kernels write dPre of every token (float32, hyperplane slot l * PE + t);
// race_dw_partial streams the rows and dPre once and leaves one partial
// [NHP][d] per workgroup; race_dw_finalize adds the partials in a fixed order.
#pragma once
#include "race_device.hpp"

namespace race {

struct DWArgs {
  const void* X0;          // query rows [BH][N][d]
  const void* X1;          // key rows [BH][N][d]
  const float* dpre0;      // dL/dPre of the query rows [BH][N][NHP]
  const float* dpre1;      // dL/dPre of the key rows [BH][N][NHP]
  float* part;             // [2][BH][nchunk][NHP][d]
  int64_t N;
  int64_t chunk_tokens;    // unused: workgroups take interleaved tiles (below)
  int nchunk;
};

constexpr int DW_TT = 128;   // tokens per tile: 32 per wave

template <typename T, int C>
struct alignas(sizeof(T) * C) ColsT {
  T v[C];
};

// grid (nchunk, BH, 2 sides), 256 threads.  Workgroup slot c takes tiles
// c, c + nchunk, c + 2 nchunk, ... (slots ordered so that each XCD takes one
// contiguous eighth of every sweep when nchunk is a multiple of 8), as the
// other streaming kernels do.  Lane owns columns
// [C * lane, C * lane + C) of d; wave w takes rows w, w + 4, ... of each tile;
// the tile's dPre rows are staged in LDS and read as broadcasts.  The next
// tile's loads are in flight while the current tile is accumulated.
template <typename T, class G>
__global__ __launch_bounds__(256) void race_dw_partial(DWArgs a) {
  constexpr int D = G::D, NHP = G::NHP, NQ = NHP / 4;
  constexpr int C = D / 64;
  constexpr int TPW = DW_TT / 4;
  constexpr int NPR = cdiv(DW_TT * NQ, 256);     // float4 of dPre per thread per tile
  static_assert(D % 64 == 0, "every lane owns whole columns");
  static_assert(NHP % 4 == 0, "dPre rows are read as float4");
  using Cols = ColsT<T, C>;
  __shared__ float4 dps[2][DW_TT * NQ];
  __shared__ float red[NHP * D];

  const int side = blockIdx.z, bh = blockIdx.y, chunk = blockIdx.x;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const T* X = static_cast<const T*>(side ? a.X1 : a.X0) + (size_t)bh * a.N * D;
  const float* dp = (side ? a.dpre1 : a.dpre0) + (size_t)bh * a.N * NHP;
  int64_t slot = chunk;
  if (a.nchunk % 8 == 0) slot = (int64_t)(chunk % 8) * (a.nchunk / 8) + chunk / 8;
  const int64_t t0 = slot * DW_TT, tstep = (int64_t)a.nchunk * DW_TT;
  const int64_t total_tiles = (a.N + DW_TT - 1) / DW_TT;   // >= nchunk > slot
  const int ntiles = (int)((total_tiles - slot + a.nchunk - 1) / a.nchunk);
  const int64_t last = a.N - 1;

  float acc[NHP][C];
#pragma unroll
  for (int i = 0; i < NHP; ++i)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[i][c] = 0.f;

  Cols xa[TPW], xc[TPW];
  float4 pa[NPR];
  // loads of the workgroup's tile k, rows clamped to the sequence (rows past
  // it get dPre = 0)
  auto load_tile = [&](int k) {
    const int64_t base = t0 + (int64_t)k * tstep;
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const int64_t r = min(base + 4 * j + w, last);
      xa[j] = *reinterpret_cast<const Cols*>(X + r * D + C * lane);
    }
#pragma unroll
    for (int i = 0; i < NPR; ++i) {
      const int idx = min((int)threadIdx.x + 256 * i, DW_TT * NQ - 1);
      const int64_t r = min(base + idx / NQ, last);
      pa[i] = *reinterpret_cast<const float4*>(dp + r * NHP + 4 * (idx % NQ));
    }
  };
  load_tile(0);
  for (int k = 0; k < ntiles; ++k) {
    const int bb = k & 1;
    const int64_t base = t0 + (int64_t)k * tstep;
#pragma unroll
    for (int i = 0; i < NPR; ++i) {
      const int idx = (int)threadIdx.x + 256 * i;
      if (idx < DW_TT * NQ) dps[bb][idx] = base + idx / NQ <= last ? pa[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) xc[j] = xa[j];
    __syncthreads();
    load_tile(min(k + 1, ntiles - 1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      float xv[C];
#pragma unroll
      for (int c = 0; c < C; ++c) xv[c] = (float)xc[j].v[c];
      const float4* drow = &dps[bb][(4 * j + w) * NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const float4 d4 = drow[q];
#pragma unroll
        for (int c = 0; c < C; ++c) {
          acc[4 * q + 0][c] += d4.x * xv[c];
          acc[4 * q + 1][c] += d4.y * xv[c];
          acc[4 * q + 2][c] += d4.z * xv[c];
          acc[4 * q + 3][c] += d4.w * xv[c];
        }
      }
    }
  }
  // waves added in a fixed order: ((w3 + w2) + w1) + w0
  for (int src = 3; src >= 0; --src) {
    if (w == src) {
#pragma unroll
      for (int i = 0; i < NHP; ++i)
#pragma unroll
        for (int c = 0; c < C; ++c) {
          float* r = &red[i * D + C * lane + c];
          *r = src == 3 ? acc[i][c] : *r + acc[i][c];
        }
    }
    __syncthreads();
  }
  float* out = a.part + (((size_t)side * gridDim.y + bh) * a.nchunk + chunk) * NHP * D;
  for (int i = threadIdx.x; i < NHP * D; i += 256) out[i] = red[i];
}

// dW[hw][l][t][c] = sum over (side, b, h, chunk) of
// part[side][b * H + h][chunk][l * PE + t][c], with h = hw for per-head
// tables and every head for shared ones; dW rows have ld <= D columns.  One workgroup per output row
// (hw, l, t): thread (c, g) adds the chunks g, g + G, ... of every (side, b,
// h) in order, then the G group sums are added in order.
static __global__ __launch_bounds__(1024) void race_dw_finalize(const float* __restrict__ part, int B, int H,
                                                                int per_head, int nchunk, int NHP, int PE, int L,
                                                                int P, int D, int ld, float* __restrict__ dW) {
  __shared__ float red[1024];
  const int row = blockIdx.x;
  const int hw = row / (L * P), lt = row % (L * P);
  const int slot = (lt / P) * PE + lt % P;
  const int c = threadIdx.x % D, g = threadIdx.x / D, G = blockDim.x / D;
  const int nh = per_head ? 1 : H, h0 = per_head ? hw : 0;
  float s = 0.f;
  for (int side = 0; side < 2; ++side)
    for (int b = 0; b < B; ++b)
      for (int hh = h0; hh < h0 + nh; ++hh) {
        const float* p = part + ((((size_t)side * B + b) * H + hh) * nchunk * NHP + slot) * D + c;
#pragma unroll 8
        for (int ch = g; ch < nchunk; ch += G) s += p[(size_t)ch * NHP * D];
      }
  red[threadIdx.x] = s;
  __syncthreads();
  if (g == 0 && c < ld) {
    float t = 0.f;
    for (int k = 0; k < G; ++k) t += red[k * D + c];
    dW[(size_t)row * ld + c] = t;
  }
}

}  // namespace race
