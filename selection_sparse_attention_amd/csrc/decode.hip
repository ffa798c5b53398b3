// Split-KV sparse decode: exact softmax attention of each query head over its
// KV group's visible set (HGA summary, Core mechanism item 4: exact attention
// over the routed tokens; "Full Attention Strikes Back" summary, Methodology
// items 1 and 5: sinks + window for local heads, bandwidth-oriented sparse
// decode for retrieval heads; S2O summary, Methodology 1 and 3: index-guided
// loading of non-contiguous rows and an online-softmax (m, l, acc) state).
//
// Grid: (split, KV group, sequence).  A workgroup takes `tps` consecutive
// entries of its group's list, gathers each K and V row exactly once and uses
// it for all G query heads of the group (GQA sharing).  A 64-lane wave works
// on 4 rows at a time, 16 lanes per row, each lane owning d/16 consecutive
// dims; it keeps 4 rows x U rounds of loads in flight before computing.  The
// (m, l, acc) state is merged across lane groups with shuffles, across waves
// through LDS, and written as a split partial.  A second launch merges each
// head's splits, every thread owning one output dim and a share of the splits.
// (Cross-workgroup merging at the kernel boundary avoids agent-scope fences,
// each of which writes back the whole L2 of its die on this chip.)  Scores use
// exp2 with log2(e)/sqrt(d) folded into the scale.
#include <type_traits>

#include "args.hpp"
#include "common.hpp"

namespace sa {

constexpr int kDecThreads = 256;
constexpr int kDecRounds = 4;        // rows in flight per lane group
constexpr int kMaxSplitsLds = 8192;  // splits merged by one combine workgroup

__device__ __forceinline__ float safe_exp2_diff(float x, float m) {
  return (x == -INFINITY) ? 0.f : exp2f(x - m);
}

template <typename T, int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int EPL = D / 16;               // elements per lane
  constexpr int U = kDecRounds;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int lg = lane >> 4, sub = lane & 15;
  const bool local = (a.local_mask >> g) & 1ull;
  const int n = a.n;
  int count, s_eff = 0, ws = 0;
  if (local) {
    s_eff = min(a.sinks, n);
    ws = max(s_eff, n - a.window);
    count = s_eff + (n - ws);
  } else {
    count = min(max(a.sel_count[(int64_t)b * a.Hkv + g], 0), n);
  }
  const int start = split * a.tps;
  if (start >= count) return;
  const int end = min(count, start + a.tps);

  float q[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
    VecLoad<T, EPL>::run(a.q, ((int64_t)b * a.Hq + g * G + h) * D + sub * EPL, q[h]);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY; l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const int64_t row0 = ((int64_t)b * a.Hkv + g) * a.n_cap;
  const int32_t* list = a.sel_idx + row0;
  const int64_t kv0 = (((int64_t)b * a.Hkv + g) / a.kv_div) * a.n_cap;
  const float sc = a.scale_log2;

  for (int base = start; base < end; base += 16 * U) {
    float kk[U][EPL], vv[U][EPL];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * 16 + wid * 4 + lg;
      valid[u] = i < end;
      int tok = 0;
      if (valid[u]) tok = local ? (i < s_eff ? i : ws + (i - s_eff)) : list[i];
      valid[u] = valid[u] && (unsigned)tok < (unsigned)n;   // ignore malformed entries
      if (valid[u]) {
        VecLoad<T, EPL>::run(a.k, (kv0 + tok) * D + sub * EPL, kk[u]);
        VecLoad<T, EPL>::run(a.v, (kv0 + tok) * D + sub * EPL, vv[u]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) { kk[u][e] = 0.f; vv[u][e] = 0.f; }
      }
    }
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) p = fmaf(q[h][e], kk[u][e], p);
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) p += __shfl_xor(p, o, 16);
        s[u][h] = valid[u] ? p * sc : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][h]);
      const float mn = fmaxf(m[h], mx);
      const float alpha = (m[h] == mn) ? 1.f : exp2f(m[h] - mn);
      float pu[U], ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) { pu[u] = safe_exp2_diff(s[u][h], mn); ps += pu[u]; }
      l[h] = l[h] * alpha + ps;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float x = acc[h][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) x = fmaf(pu[u], vv[u][e], x);
        acc[h][e] = x;
      }
      m[h] = mn;
    }
  }

  // merge the four lane groups of the wave
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float M = fmaxf(m[h], mo);
      const float wa = safe_exp2_diff(m[h], M), wb = safe_exp2_diff(mo, M);
      l[h] = l[h] * wa + lo * wb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[h][e], off);
        acc[h][e] = acc[h][e] * wa + ao * wb;
      }
      m[h] = M;
    }
  }
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_acc[4][G][D];
  if (lg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wid][h][sub * EPL + e] = acc[h][e];
      if (sub == 0) { s_m[wid][h] = m[h]; s_l[wid][h] = l[h]; }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kDecThreads) {
    const int h = idx / D, e = idx % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
    float av = 0.f, lv = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = safe_exp2_diff(s_m[w][h], M);
      av += wt * s_acc[w][h][e];
      lv += wt * s_l[w][h];
    }
    float* pp = a.partial + (((int64_t)b * a.Hq + g * G + h) * a.max_splits + split) * (D + 2);
    pp[e] = av;
    if (e == 0) { pp[D] = M; pp[D + 1] = lv; }
  }
}

// Merge the splits of one (sequence, query head): weights 2^(m_s - M) per
// split, then every thread sums one output dim over its share of the splits.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  constexpr int P = 256 / D;                 // split shares per output dim
  __shared__ float s_w[kMaxSplitsLds];
  __shared__ float s_red[256];
  __shared__ float s_M, s_L;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq, g = h / a.G;
  int count;
  if ((a.local_mask >> g) & 1ull) {
    const int s_eff = min(a.sinks, a.n);
    count = s_eff + (a.n - max(s_eff, a.n - a.window));
  } else {
    count = min(max(a.sel_count[(int64_t)b * a.Hkv + g], 0), a.n);
  }
  const int ns = (count + a.tps - 1) / a.tps;
  const float* base = a.partial + (int64_t)bh * a.max_splits * (D + 2);
  float mx = -INFINITY;
  for (int sp = tid; sp < ns; sp += 256) mx = fmaxf(mx, base[(int64_t)sp * (D + 2) + D]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) s_red[tid >> 6] = mx;
  __syncthreads();
  if (tid == 0) s_M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  const float M = s_M;
  float lsum = 0.f;
  for (int sp = tid; sp < ns; sp += 256) {
    const float* q = base + (int64_t)sp * (D + 2);
    const float w = (q[D] == -INFINITY) ? 0.f : exp2f(q[D] - M);
    s_w[sp] = w;
    lsum += w * q[D + 1];
  }
  lsum = wave_sum(lsum);
  __syncthreads();
  if ((tid & 63) == 0) s_red[tid >> 6] = lsum;
  __syncthreads();
  if (tid == 0) s_L = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  __syncthreads();
  const int e = tid % D, part = tid / D;
  float acc = 0.f;
#pragma unroll 8
  for (int sp = part; sp < ns; sp += P) acc = fmaf(s_w[sp], base[(int64_t)sp * (D + 2) + e], acc);
  s_red[tid] = acc;
  __syncthreads();
  if (part == 0) {
    float v = acc;
#pragma unroll
    for (int q = 1; q < P; ++q) v += s_red[q * D + e];
    const float L = s_L;
    // a failed selection (negative count) poisons the group's outputs
    const bool failed = !((a.local_mask >> g) & 1ull) && a.sel_count[(int64_t)b * a.Hkv + g] < 0;
    a.out[(int64_t)bh * D + e] = failed ? __builtin_nanf("") : ((L > 0.f) ? v / L : 0.f);
  }
}

template <typename T, int D>
static hipError_t run_decode(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.max_splits, a.Hkv, a.B);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<T, D, 1>), grid, dim3(kDecThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<T, D, 2>), grid, dim3(kDecThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<T, D, 4>), grid, dim3(kDecThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_split_kernel<T, D, 8>), grid, dim3(kDecThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  if (a.max_splits > kMaxSplitsLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.Hq), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, hipStream_t s) {
  if (dtype == 0) return launch_decode_mfma(a, d, s);      // bf16 caches: matrix-core path
  if (dtype == 1 && d == 128) return run_decode<float, 128>(a, s);
  if (dtype == 1 && d == 64) return run_decode<float, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace sa
