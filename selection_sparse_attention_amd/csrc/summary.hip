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
// One 256-thread workgroup per (span, KV group, sequence), four threads per
// pair; the x-range of the grid covers the chunks first, then the groups.
#include "args.hpp"
#include "common.hpp"

namespace sa {

constexpr int kSumThreads = 256;
constexpr int kSumParts = kSumThreads / 64;     // token quarters of a span

// Thread (pair i, part q) of a 64-pair workgroup layout: pair i of the span's
// tokens q, q + 4, q + 8, ...; the four partial sums meet in LDS.  A
// high-frequency pair's angle advances by theta per token through an exact
// fp64 rotation recurrence (one sincos per thread instead of one per token).
template <typename T, int D>
__global__ __launch_bounds__(kSumThreads) void summary_kernel(SummaryArgs a) {
  constexpr int H = D / 2;
  __shared__ double s_x[kSumParts][64], s_y[kSumParts][64];
  const int nch = a.c1 - a.c0;
  const int x = blockIdx.x, gi = blockIdx.y, b = blockIdx.z;
  const int g = a.groups.ids[gi];
  const bool is_chunk = x < nch;
  const int span = is_chunk ? a.chunk : a.group;
  const int idx = is_chunk ? a.c0 + x : a.g0 + (x - nch);
  const int64_t rows_per_bg = is_chunk ? (a.n_cap / a.chunk) : (a.n_cap / a.group);
  void* dst = is_chunk ? a.chunk_sum : a.group_sum;
  const int64_t drow = (((int64_t)b * a.Hkv + g) * rows_per_bg + idx) * D;
  const int i = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int start = idx * span;
  const int64_t krow = ((int64_t)b * a.Hkv + g) * a.n_cap;
  double sx = 0.0, sy = 0.0;
  double theta = 0.0;
  bool high = false;
  if (i < H) {
    theta = pow(a.rope_base, -2.0 * (double)i / (double)D);
    high = theta * (double)(span - 1) > 1.0;
    double c = 1.0, sn = 0.0, cs = 1.0, ss = 0.0;
    if (high) {
      sincos((double)(start + q) * theta, &sn, &c);     // angle of this thread's first token
      sincos((double)kSumParts * theta, &ss, &cs);      // advance per step
    }
    for (int j0 = q; j0 < span; j0 += 4 * kSumParts) {
      float xv[4], yv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {                     // loads of four steps in flight
        const int jj = j0 + u * kSumParts;
        const int p = start + min(jj, span - 1);
        xv[u] = Elem<T>::load(a.k_pre, (krow + p) * D + i);
        yv[u] = Elem<T>::load(a.k_pre, (krow + p) * D + i + H);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j0 + u * kSumParts < span) {
          const double xd = xv[u], yd = yv[u];
          if (high) {
            sx += xd * c - yd * sn;
            sy += xd * sn + yd * c;
            const double c2 = c * cs - sn * ss, s2 = sn * cs + c * ss;
            c = c2;
            sn = s2;
          } else {
            sx += xd;
            sy += yd;
          }
        }
      }
    }
  }
  s_x[q][i] = sx;
  s_y[q][i] = sy;
  __syncthreads();
  if (q != 0 || i >= H) return;
  sx = s_x[0][i] + s_x[1][i] + s_x[2][i] + s_x[3][i];
  sy = s_y[0][i] + s_y[1][i] + s_y[2][i] + s_y[3][i];
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
  Elem<T>::store_d(dst, drow + i + H, sy);
}

hipError_t launch_summary(const SummaryArgs& a, int dtype, int d, hipStream_t s) {
  const int nx = (a.c1 - a.c0) + (a.g1 - a.g0);
  if (nx <= 0 || a.groups.n == 0) return hipSuccess;
  dim3 grid(nx, a.groups.n, a.B), block(kSumThreads);
  if (dtype == 0 && d == 128) hipLaunchKernelGGL((summary_kernel<bf16_t, 128>), grid, block, 0, s, a);
  else if (dtype == 0 && d == 64) hipLaunchKernelGGL((summary_kernel<bf16_t, 64>), grid, block, 0, s, a);
  else if (dtype == 1 && d == 128) hipLaunchKernelGGL((summary_kernel<float, 128>), grid, block, 0, s, a);
  else if (dtype == 1 && d == 64) hipLaunchKernelGGL((summary_kernel<float, 64>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
