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

template <int D, int U, int NT, typename Store>
__device__ __forceinline__ void project_rows_mfma_st(const void* src, const float* Pg, int64_t row0,
                                                     int first, int last, Store st) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int col = lane & 15, kb = lane >> 4;
  const uint16_t* sp = reinterpret_cast<const uint16_t*>(src);
  constexpr int STEP = 16 * U * (NT / 64);            // rows per workgroup step
  auto load_rows = [&](int base, vl_u32x4 (&av)[U][KS]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(base + 16 * u + col, last - 1);
#pragma unroll
      for (int s = 0; s < KS; ++s)
        av[u][s] = __builtin_nontemporal_load(
            reinterpret_cast<const vl_u32x4*>(sp + (row0 + r) * D + 32 * s + 8 * kb));
    }
  };
  // the first step's rows are requested before the projector is loaded and
  // split, so the two memory latencies overlap (an append is one step)
  int base = first + wid * 16 * U;
  vl_u32x4 av[U][KS];
  if (base < last) load_rows(base, av);
  ix_bf16x8 ph[KS], pm[KS], pl[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const float* pr = Pg + col * D + 32 * s + 8 * kb;
    const vl_f32x4 x0 = *reinterpret_cast<const vl_f32x4*>(pr);
    const vl_f32x4 x1 = *reinterpret_cast<const vl_f32x4*>(pr + 4);
    float p[8], r1[8], r2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = i < 4 ? x0[i] : x1[i - 4];
    // p = hi + mid + lo, each part the nearest bf16 of what is left
    // (v_cvt_pk_bf16_f32 rounds to nearest even)
    ix_bf16x8 h, m, l;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (__bf16)p[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) r1[i] = p[i] - (float)h[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = (__bf16)r1[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) r2[i] = r1[i] - (float)m[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) l[i] = (__bf16)r2[i];
    ph[s] = h;
    pm[s] = m;
    pl[s] = l;
  }
  for (; base < last; base += STEP) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ix_f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const ix_bf16x8 av8 = __builtin_bit_cast(ix_bf16x8, av[u][s]);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av8, pl[s], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av8, pm[s], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av8, ph[s], c, 0, 0, 0);
      }
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
