// Low-rank pre-RoPE token index ("Full Attention Strikes Back" summary,
// Methodology item 2): a 16-dim projector is applied to the query and key
// features before RoPE, and relevance is later estimated in that subspace.
//
// k_idx[b,g,j,c] = sum_e P_k[g,c,e] * k_pre[b,g,j,e]   (fp32, rounded once)
// q_idx[b,h,c]   = sum_e P_q[g,c,e] * q_pre[b,h,e]     (fp32)
//
// One workgroup projects 16 tokens of one (sequence, retrieval group): the
// group's projector (16 x d fp32) and the 16 key rows are staged in LDS and
// each of the 256 threads produces one (token, component) output.  The last
// x-block of the grid projects the group's query heads instead.  This is an
// HBM-bound pass over k_pre (d * e bytes per token in, 16 * e out).
#include "args.hpp"
#include "common.hpp"

namespace sa {

template <typename T, int D>
__global__ __launch_bounds__(256) void index_lowrank_kernel(IndexLowrankArgs a) {
  __shared__ float sP[16][D + 1];
  __shared__ float sK[16][D + 1];
  const int tid = threadIdx.x;
  const int gi = blockIdx.y, b = blockIdx.z;
  const int g = a.groups.ids[gi];
  const int ntiles = (a.t1 - a.t0 + 15) / 16;
  const bool q_side = (int)blockIdx.x == ntiles;
  const float* P = (q_side ? a.proj_q : a.proj_k) + (int64_t)g * 16 * D;

  for (int i = tid; i < 16 * D; i += 256) sP[i / D][i % D] = P[i];

  if (q_side) {
    if (a.q_pre == nullptr) return;
    __syncthreads();
    // 16 heads per pass of the workgroup, as many passes as the group has heads
    const int c = tid % 16;
    for (int hh = tid / 16; hh < a.G; hh += 16) {
      const int h = g * a.G + hh;
      const int64_t base = ((int64_t)b * a.Hq + h) * D;
      float acc = 0.f;
      for (int e = 0; e < D; ++e) acc = fmaf(sP[c][e], Elem<T>::load(a.q_pre, base + e), acc);
      a.q_idx[((int64_t)b * a.Hq + h) * 16 + c] = acc;
    }
    return;
  }

  const int j0 = a.t0 + 16 * blockIdx.x;
  const int64_t row0 = ((int64_t)b * a.Hkv + g) * a.n_cap;
  for (int i = tid; i < 16 * D; i += 256) {
    const int jj = i / D, e = i % D;
    const int j = j0 + jj;
    sK[jj][e] = (j < a.t1) ? Elem<T>::load(a.k_pre, (row0 + j) * D + e) : 0.f;
  }
  __syncthreads();
  const int jj = tid / 16, c = tid % 16;
  const int j = j0 + jj;
  if (j >= a.t1) return;
  float acc = 0.f;
#pragma unroll 8
  for (int e = 0; e < D; ++e) acc = fmaf(sP[c][e], sK[jj][e], acc);
  Elem<T>::store(a.k_idx, (row0 + j) * 16 + c, acc);
}

hipError_t launch_index_lowrank(const IndexLowrankArgs& a, int dtype, int d, hipStream_t s) {
  const int ntiles = (a.t1 - a.t0 + 15) / 16;
  dim3 grid(ntiles + 1, a.groups.n, a.B);
  if (dtype == 0 && d == 128) hipLaunchKernelGGL((index_lowrank_kernel<bf16_t, 128>), grid, dim3(256), 0, s, a);
  else if (dtype == 0 && d == 64) hipLaunchKernelGGL((index_lowrank_kernel<bf16_t, 64>), grid, dim3(256), 0, s, a);
  else if (dtype == 1 && d == 128) hipLaunchKernelGGL((index_lowrank_kernel<float, 128>), grid, dim3(256), 0, s, a);
  else if (dtype == 1 && d == 64) hipLaunchKernelGGL((index_lowrank_kernel<float, 64>), grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
