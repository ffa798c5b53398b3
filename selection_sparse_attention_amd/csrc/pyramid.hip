// Symmetric mean pyramid over Q, K, V and the parameter-free entry scores
// (Lighthouse summary, Methodology 2A and 2B).
//
// Level 0 is the full-resolution sequence; an entry of level l is the mean of
// p consecutive entries of level l-1, i.e. of its p^l level-0 rows.  Each
// stored coarse entry is that exact mean (accumulated in fp64) rounded once to
// the element type.  The score of a level-0 entry is |q|^2 + |k|^2 (the
// squared l2 norm of the projected query and key: the ranking the norm gives);
// a coarse entry inherits the largest score among the entries it covers.
//
// One workgroup (d threads, one per dim) per span of p^(L-1) level-0 rows of
// one (sequence, head): it streams the span once, 16 rows' loads in flight at
// a time, emits every coarse entry of every level inside it, and the span's
// scores.
#include "args.hpp"
#include "common.hpp"

namespace sa {

// Sum over the 64 lanes of a wave: DPP rotations inside each 16-lane row,
// then two cross-row exchanges.
__device__ __forceinline__ float wave_sum_rows(float v) {
  v += dpp_move<0x128, 0xF>(v);     // row_ror:8
  v += dpp_move<0x124, 0xF>(v);     // row_ror:4
  v += dpp_move<0x122, 0xF>(v);     // row_ror:2
  v += dpp_move<0x121, 0xF>(v);     // row_ror:1
  v += __shfl_xor(v, 32);
  v += __shfl_xor(v, 16);
  return v;
}

template <typename T, int D>
__global__ __launch_bounds__(D) void pyramid_kernel(PyramidArgs a) {
  constexpr int NW = D / 64;
  __shared__ float s_part[NW][256];
  __shared__ float s_score[256];
  const int span = blockIdx.x, bh = blockIdx.y, e = threadIdx.x;
  const int lane = e & 63, wid = e >> 6;
  const int P = a.top_span;
  const int64_t r0 = (int64_t)span * P;                  // first level-0 row
  const int64_t base = (int64_t)bh * a.N + r0;
  double aq[8], ak[8], av[8];
#pragma unroll
  for (int l = 0; l < 8; ++l) { aq[l] = 0.0; ak[l] = 0.0; av[l] = 0.0; }
  // per level: rows per entry, rows still to add to the open entry, and the
  // index of that entry inside the level (no division per row)
  int ewidth[8], left[8];
  int64_t jnext[8];
  double inv[8];
  {
    int w = 1;
#pragma unroll
    for (int l = 1; l < 8; ++l) {
      w = (l < a.levels) ? w * a.factor : w;
      ewidth[l] = w;
      left[l] = w;
      jnext[l] = r0 / w;
      inv[l] = 1.0 / (double)w;
    }
  }
  // rows in batches of kRows: every load of a batch is issued before any is
  // used (rows past the span re-read its last row and are skipped)
  constexpr int kRows = 16;
  for (int rb = 0; rb < P; rb += kRows) {
    float xq[kRows], xk[kRows], xv[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int64_t r = base + min(rb + u, P - 1);
      xq[u] = Elem<T>::load(a.q, r * D + e);
      xk[u] = Elem<T>::load(a.k, r * D + e);
      xv[u] = Elem<T>::load(a.v, r * D + e);
    }
    float sq[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u) sq[u] = xq[u] * xq[u] + xk[u] * xk[u];
#pragma unroll
    for (int u = 0; u < kRows; ++u) sq[u] = wave_sum_rows(sq[u]);
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int r = rb + u;
      if (r >= P) break;
      if (lane == 0) s_part[wid][r] = sq[u];
#pragma unroll
      for (int l = 1; l < 8; ++l) {
        if (l >= a.levels) break;
        aq[l] += xq[u]; ak[l] += xk[u]; av[l] += xv[u];
        if (--left[l] == 0) {                           // entry jnext[l] of level l is complete
          const int64_t row = (int64_t)bh * a.Nc + a.coff[l] + jnext[l];
          Elem<T>::store_d(a.pq, row * D + e, aq[l] * inv[l]);
          Elem<T>::store_d(a.pk, row * D + e, ak[l] * inv[l]);
          Elem<T>::store_d(a.pv, row * D + e, av[l] * inv[l]);
          aq[l] = 0.0; ak[l] = 0.0; av[l] = 0.0;
          left[l] = ewidth[l];
          ++jnext[l];
        }
      }
    }
  }
  __syncthreads();
  float* sc = a.scores + (int64_t)bh * a.Nt;
  for (int r = e; r < P; r += D) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += s_part[w][r];
    s_score[r] = s;
    sc[r0 + r] = s;
  }
  __syncthreads();
  // coarse scores: the max over each entry's level-0 rows
  int width = 1;
  for (int l = 1; l < a.levels; ++l) {
    width *= a.factor;
    const int cnt = P / width;
    for (int j = e; j < cnt; j += D) {
      float m = s_score[j * width];
      for (int r = 1; r < width; ++r) m = fmaxf(m, s_score[j * width + r]);
      sc[a.soff[l] + r0 / width + j] = m;
    }
  }
}

hipError_t launch_pyramid(const PyramidArgs& a, int dtype, int d, hipStream_t s) {
  if (a.top_span > 256 || a.levels > 8) return hipErrorInvalidValue;
  dim3 grid(a.N / a.top_span, a.B * a.H);
  if (dtype == 0 && d == 128) hipLaunchKernelGGL((pyramid_kernel<bf16_t, 128>), grid, dim3(128), 0, s, a);
  else if (dtype == 0 && d == 64) hipLaunchKernelGGL((pyramid_kernel<bf16_t, 64>), grid, dim3(64), 0, s, a);
  else if (dtype == 1 && d == 128) hipLaunchKernelGGL((pyramid_kernel<float, 128>), grid, dim3(128), 0, s, a);
  else if (dtype == 1 && d == 64) hipLaunchKernelGGL((pyramid_kernel<float, 64>), grid, dim3(64), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
