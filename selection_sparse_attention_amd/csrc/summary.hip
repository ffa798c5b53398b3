// RoPE-aware chunk and group key summaries (HGA summary, Core mechanism
// item 3): summaries are built from the existing pre-RoPE keys with no new
// weights, using a mixed rule per RoPE pair - high-frequency pairs are rotated
// to each token's position and then averaged, low-frequency pairs are averaged
// in raw key space and rotated once at the span's representative position.
//
// Pair i couples dims i and i + d/2 and turns by theta_i = base^(-2i/d) per
// position.  Pair i counts as high-frequency when theta_i * (span - 1) > 1
// rad (over one span it turns by more than a radian); the representative
// position is the span's mean position start + (span - 1)/2.  Angles, the
// rotation and the average are formed in fp64 and rounded once to the
// summary element type.
//
// One 64-thread workgroup per (span, KV group, sequence), one thread per
// pair; the x-range of the grid covers the chunks first, then the groups.
#include "args.hpp"
#include "common.hpp"

namespace sa {

template <typename T, int D>
__global__ __launch_bounds__(64) void summary_kernel(SummaryArgs a) {
  const int nch = a.c1 - a.c0;
  const int x = blockIdx.x, gi = blockIdx.y, b = blockIdx.z;
  const int g = a.groups.ids[gi];
  const bool is_chunk = x < nch;
  const int span = is_chunk ? a.chunk : a.group;
  const int idx = is_chunk ? a.c0 + x : a.g0 + (x - nch);
  const int64_t rows_per_bg = is_chunk ? (a.n_cap / a.chunk) : (a.n_cap / a.group);
  void* dst = is_chunk ? a.chunk_sum : a.group_sum;
  const int64_t drow = (((int64_t)b * a.Hkv + g) * rows_per_bg + idx) * D;
  const int i = threadIdx.x;
  if (i >= D / 2) return;
  const int start = idx * span;
  const double theta = pow(a.rope_base, -2.0 * (double)i / (double)D);
  const bool high = theta * (double)(span - 1) > 1.0;
  const int64_t krow = ((int64_t)b * a.Hkv + g) * a.n_cap;
  double sx = 0.0, sy = 0.0;
  for (int jj = 0; jj < span; ++jj) {
    const int p = start + jj;
    const double xv = Elem<T>::load(a.k_pre, (krow + p) * D + i);
    const double yv = Elem<T>::load(a.k_pre, (krow + p) * D + i + D / 2);
    if (high) {
      double sn, cs;
      sincos((double)p * theta, &sn, &cs);
      sx += xv * cs - yv * sn;
      sy += xv * sn + yv * cs;
    } else {
      sx += xv;
      sy += yv;
    }
  }
  sx /= (double)span;
  sy /= (double)span;
  if (!high) {
    double sn, cs;
    sincos(((double)start + 0.5 * (double)(span - 1)) * theta, &sn, &cs);
    const double rx = sx * cs - sy * sn, ry = sx * sn + sy * cs;
    sx = rx;
    sy = ry;
  }
  Elem<T>::store_d(dst, drow + i, sx);
  Elem<T>::store_d(dst, drow + i + D / 2, sy);
}

hipError_t launch_summary(const SummaryArgs& a, int dtype, int d, hipStream_t s) {
  const int nx = (a.c1 - a.c0) + (a.g1 - a.g0);
  if (nx <= 0 || a.groups.n == 0) return hipSuccess;
  dim3 grid(nx, a.groups.n, a.B), block(64);
  if (dtype == 0 && d == 128) hipLaunchKernelGGL((summary_kernel<bf16_t, 128>), grid, block, 0, s, a);
  else if (dtype == 0 && d == 64) hipLaunchKernelGGL((summary_kernel<bf16_t, 64>), grid, block, 0, s, a);
  else if (dtype == 1 && d == 128) hipLaunchKernelGGL((summary_kernel<float, 128>), grid, block, 0, s, a);
  else if (dtype == 1 && d == 64) hipLaunchKernelGGL((summary_kernel<float, 64>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
