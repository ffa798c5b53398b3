// Low-rank projection of bf16 rows on the matrix cores ("Full Attention
// Strikes Back" summary, Methodology item 2: a 16-dim projector applied to
// the pre-RoPE query and key features).  Shared by the index build and the
// selector's fused append, so that both produce the same bits for a row.
#pragma once

#include "common.hpp"

namespace sa {

// bf16 rows on the matrix cores: for a tile of 16 rows, out[row][c] =
// sum_e row[e] P[c][e] is one v_mfma_f32_16x16x32_bf16 per 32 dims, with the
// rows as the A operand (lane l: row l % 16, dims 32 s + 8 (l / 16) .. +8, 64
// contiguous bytes of every row per load) and the projector as the B operand
// (lane l: output l % 16, the same dims).  The fp32 projector is split into
// three bf16 parts (p = hi + mid + lo up to 2^-24 |p|), each multiplied in, so
// the sum keeps fp32's precision; the accumulation is fp32.  The result
// leaves rows 4 (l / 16) .. +4 of output l % 16 on lane l, handed to
// st(row, output, value) for every row below `last` (rows row0 + first ..
// row0 + last - 1 of src; NT threads, the workgroup, take part).
typedef __bf16 ix_bf16x8 __attribute__((ext_vector_type(8)));
typedef float ix_f32x4 __attribute__((ext_vector_type(4)));

// This lane's slices of the fp32 projector (output l % 16, dims 32 s + 8 (l /
// 16) .. +8), as loaded.
template <int D>
struct ProjSlices {
  vl_f32x4 x[D / 32][2];
  __device__ __forceinline__ void load(const float* Pg) {
    const int lane = threadIdx.x & 63, col = lane & 15, kb = lane >> 4;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const float* pr = Pg + col * D + 32 * s + 8 * kb;
      x[s][0] = *reinterpret_cast<const vl_f32x4*>(pr);
      x[s][1] = *reinterpret_cast<const vl_f32x4*>(pr + 4);
    }
  }
};

// The projector as the B operand: p = hi + mid + lo, each part the nearest
// bf16 of what is left (v_cvt_pk_bf16_f32 rounds to nearest even).
template <int D>
struct ProjParts {
  ix_bf16x8 h[D / 32], m[D / 32], l[D / 32];
  __device__ __forceinline__ void split(const ProjSlices<D>& ps) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      float p[8], r1[8], r2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = i < 4 ? ps.x[s][0][i] : ps.x[s][1][i - 4];
      ix_bf16x8 hh, mm, ll;
#pragma unroll
      for (int i = 0; i < 8; ++i) hh[i] = (__bf16)p[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) r1[i] = p[i] - (float)hh[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) mm[i] = (__bf16)r1[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) r2[i] = r1[i] - (float)mm[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) ll[i] = (__bf16)r2[i];
      h[s] = hh;
      m[s] = mm;
      l[s] = ll;
    }
  }
  // one tile: the row slices of this lane (row l % 16) times the projector,
  // the lo, mid and hi parts in turn for each 32 dims
  __device__ __forceinline__ ix_f32x4 tile(const vl_u32x4 (&av)[D / 32]) const {
    ix_f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const ix_bf16x8 av8 = __builtin_bit_cast(ix_bf16x8, av[s]);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av8, l[s], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av8, m[s], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av8, h[s], c, 0, 0, 0);
    }
    return c;
  }
};

// This lane's slices of row min(first + l % 16, last - 1) of src (row r at
// element (row0 + r) * D): 64 contiguous bytes of the row per load.
template <int D>
__device__ __forceinline__ void load_row_slices(const void* src, int64_t row0, int first, int last,
                                                vl_u32x4 (&av)[D / 32]) {
  const int lane = threadIdx.x & 63, col = lane & 15, kb = lane >> 4;
  const uint16_t* sp = reinterpret_cast<const uint16_t*>(src);
  const int r = min(first + col, last - 1);
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    av[s] = __builtin_nontemporal_load(reinterpret_cast<const vl_u32x4*>(sp + (row0 + r) * D + 32 * s + 8 * kb));
}

template <int D, int U, int NT, typename Store>
__device__ __forceinline__ void project_rows_mfma_st(const void* src, const float* Pg, int64_t row0,
                                                     int first, int last, Store st) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int col = lane & 15, kb = lane >> 4;
  constexpr int STEP = 16 * U * (NT / 64);            // rows per workgroup step
  auto load_rows = [&](int base, vl_u32x4 (&av)[U][KS]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) load_row_slices<D>(src, row0, base + 16 * u, last, av[u]);
  };
  // the first step's rows are requested before the projector is loaded and
  // split, so the two memory latencies overlap (an append is one step)
  int base = first + wid * 16 * U;
  vl_u32x4 av[U][KS];
  if (base < last) load_rows(base, av);
  ProjSlices<D> ps;
  ps.load(Pg);
  ProjParts<D> pp;
  pp.split(ps);
  for (; base < last; base += STEP) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const ix_f32x4 c = pp.tile(av[u]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = base + 16 * u + 4 * kb + i;
        if (r < last) st(r, col, c[i]);
      }
    }
    if (base + STEP < last) load_rows(base + STEP, av);
  }
}

}  // namespace sa
