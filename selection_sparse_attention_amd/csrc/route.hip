// Two-level routing of the decode query over chunk and group key summaries
// (HGA summary, Core mechanism item 2).
//
// For each (sequence b, routed KV group g), with t = n - 1 and kappa = t / C:
//   * qbar = mean of the group's post-RoPE query heads;
//   * level 1: every complete chunk c in [sink_chunks, kappa - local_chunks)
//     is scored by qbar . chunk_sum[c]; the top_chunks highest (ties to the
//     lower chunk) are kept;
//   * level 2: inside each kept chunk the top_groups groups by
//     qbar . group_sum (ties to the lower group);
//   * the visible list is the union of the sink chunks [0, sink_chunks), the
//     local chunks [kappa - local_chunks, kappa), the current chunk's tokens
//     kappa*C .. t, and the routed groups' tokens - written ascending.
// Scores are ranked on the raw dot product: dividing by sqrt(d) does not
// change the order.
//
// One 1024-thread workgroup per (KV group, sequence): there are fewer of these
// than compute units, so each takes a whole unit and keeps as many summary
// rows in flight as it can.  Rows are scored with 16 lanes each (d/16
// elements per lane, a 16-lane DPP reduction, eight rounds of loads in
// flight), chunk scores stay in LDS, and the top chunks come from per-wave
// arg-max rounds over (score key, inverted index) 64-bit keys merged by one
// wave - no block barrier per extracted chunk.
#include <algorithm>

#include "args.hpp"
#include "common.hpp"

namespace sa {

constexpr int kRouteThreads = 1024;
constexpr int kMaxRoutedGroups = 4096;     // top_chunks * top_groups

template <int CTRL>
__device__ __forceinline__ float rdpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum_r(float v) {
  v += rdpp<0x128>(v);
  v += rdpp<0x124>(v);
  v += rdpp<0x122>(v);
  v += rdpp<0x121>(v);
  return v;
}

// Scores qbar . rows[r] for r in [0, nrows) into out[r]; rows are d wide,
// and q holds this lane's d/16 elements of qbar (lane l: elements
// (l % 16) d/16 ..). A wave scores 4 rows per round (16 lanes per row) and
// keeps the loads of U rounds in flight.
template <typename T, int D>
__device__ void score_rows(const void* base, int64_t row_of0, int nrows, const float (&q)[D / 16],
                           float* out, const int* row_map) {
  constexpr int EPL = D / 16;
  constexpr int U = 8;
  constexpr int NW = kRouteThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int sub = lane & 15, rg = lane >> 4;
  for (int r0 = 0; r0 < nrows; r0 += 4 * NW * U) {
    float kv[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = min(r0 + u * 4 * NW + wid * 4 + rg, nrows - 1);
      const int64_t row = row_map ? (int64_t)row_map[r] : (row_of0 + r);
      VecLoad<T, EPL>::run(base, row * D + sub * EPL, kv[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = r0 + u * 4 * NW + wid * 4 + rg;
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(q[e], kv[u][e], p);
      p = row16_sum_r(p);
      if (r < nrows && sub == 0) out[r] = p;
    }
  }
}

__device__ __forceinline__ uint64_t score_key(float s, int idx) {
  if (s == 0.f) s = 0.f;
  return ((uint64_t)order_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

// Largest 64-bit key over the wave (DPP max scan, then lane 63's value).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_move<0x111, 0xF>(v); v = o > v ? o : v;     // row_shr:1
  o = dpp_move<0x112, 0xF>(v); v = o > v ? o : v;     // row_shr:2
  o = dpp_move<0x114, 0xF>(v); v = o > v ? o : v;     // row_shr:4
  o = dpp_move<0x118, 0xF>(v); v = o > v ? o : v;     // row_shr:8
  o = dpp_move<0x142, 0xA>(v); v = o > v ? o : v;     // row_bcast:15
  o = dpp_move<0x143, 0xC>(v); v = o > v ? o : v;     // row_bcast:31
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one 64-bit key per lane across the wave, largest in lane 0.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, j);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), j);
      const uint64_t o = ((uint64_t)hi << 32) | lo;
      // within blocks of k lanes (all descending at the last stage) the
      // lower lane of a pair keeps the larger key
      const bool keep_max = ((lane & k) == 0) == ((lane & j) == 0);
      v = keep_max ? (o > v ? o : v) : (o < v ? o : v);
    }
  }
  return v;
}

template <typename T, int D>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
  extern __shared__ float dyn[];                 // chunk scores, then group scores
  __shared__ int s_chunks[256], s_sorted[256];
  __shared__ uint64_t s_wtop[kRouteThreads / 64][64];
  __shared__ int s_groups[kMaxRoutedGroups];
  __shared__ int s_rowmap[kMaxRoutedGroups];
  // decode: one row per (group, sequence); prefill: one per (query block,
  // group, sequence), the block's last position taking the query's place
  const int blk = blockIdx.x, gi = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int g = a.groups.ids[gi];
  const int n = a.n, C = a.chunk, GR = a.group, gpc = C / GR;
  const int t = a.prefill ? min(n, (blk + 1) * C) - 1 : n - 1;
  const int kappa = t / C;
  const int c_lo = a.sink_chunks;
  const int c_hi = max(c_lo, kappa - a.local_chunks);
  const int ncand = c_hi - c_lo;
  const int nT = min(a.top_chunks, ncand);
  const int TG = a.top_groups;

  // this lane's share of qbar, in registers (its loads overlap the first
  // summary rows' loads: no barrier in between)
  constexpr int EPL = D / 16;
  float qv[EPL];
  if (a.prefill) {
    // the block's chunk-level query: the sum of its G x nq query rows
    // (ranking by a positive multiple of the mean is ranking by the mean);
    // thread (row slot tid / 16, sub) sums every 64th row, the four row
    // slots of a wave are added by lane swaps, the 16 waves through LDS
    const int sub = tid & 15, slot = tid >> 4;
    const int q0 = blk * C, nq = t + 1 - q0, rows = a.G * nq;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = 0.f;
    for (int r = slot; r < rows; r += kRouteThreads / 16) {
      const int h = r / nq, i = r - h * nq;
      float x[EPL];
      VecLoad<T, EPL>::run(a.q, (((int64_t)b * a.Hq + g * a.G + h) * a.n + q0 + i) * D + sub * EPL, x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      qv[e] += __shfl_xor(qv[e], 16);
      qv[e] += __shfl_xor(qv[e], 32);
    }
    float (*part)[D] = reinterpret_cast<float (*)[D]>(&s_wtop[0][0]);   // [16][D]: 8 KB at D = 128
    const int lane = tid & 63, wid = tid >> 6;
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) part[wid][sub * EPL + e] = qv[e];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float x = 0.f;
      for (int w = 0; w < kRouteThreads / 64; ++w) x += part[w][sub * EPL + e];
      qv[e] = x;
    }
    __syncthreads();
  } else {
    const int sub = tid & 15;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] = 0.f;
    for (int h = 0; h < a.G; ++h) {
      float x[EPL];
      VecLoad<T, EPL>::run(a.q, ((int64_t)b * a.Hq + g * a.G + h) * D + sub * EPL, x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[e] += x[e];
    }
    const float invG = 1.0f / (float)a.G;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[e] *= invG;
  }

  const int64_t bg = (int64_t)b * a.Hkv + g;
  const int64_t kvg = bg / a.kv_div;        // the summaries' KV group
  if (nT > 0) {
    score_rows<T, D>(a.chunk_sum, kvg * a.n_cs_cap + c_lo, ncand, qv, dyn, nullptr);
    __syncthreads();
    if (nT <= 16 && ncand <= kRouteThreads) {
      // level 1 with at most one candidate per thread: every wave sorts its
      // 64 (score key, inverted index) keys, four waves sort the waves' top
      // 16s four waves at a time, and one wave the four results
      const int lane = tid & 63, wid = tid >> 6;
      uint64_t k1 = tid < ncand ? score_key(dyn[tid], tid) : 0ull;     // keys are never 0
      k1 = wave_sort_desc(k1, lane);
      if (lane < 16) s_wtop[wid][lane] = k1;
      __syncthreads();
      uint64_t k2 = 0;
      if (wid < 4) k2 = wave_sort_desc(s_wtop[4 * wid + (lane >> 4)][lane & 15], lane);
      __syncthreads();
      if (wid < 4 && lane < 16) s_wtop[wid][lane] = k2;
      __syncthreads();
      if (wid == 0) {
        const uint64_t k3 = wave_sort_desc(s_wtop[lane >> 4][lane & 15], lane);
        if (lane < nT) s_chunks[lane] = c_lo + (int)(0xFFFFFFFFu - (uint32_t)k3);
      }
    } else {
    // level 1: every wave extracts the top nT of its candidates (i = tid +
    // kRouteThreads k) by nT rounds of wave arg-max over (score key, inverted
    // index) keys; wave 0 then takes the top nT of those in order
      const int lane = tid & 63, wid = tid >> 6;
      uint64_t done_mask = 0;                        // bit k: candidate tid + kRouteThreads k taken
      for (int r = 0; r < nT; ++r) {
        uint64_t best = 0;
        for (int k = 0, i = tid; i < ncand; ++k, i += kRouteThreads)
          if (!((done_mask >> k) & 1ull)) {
            const uint64_t key = score_key(dyn[i], i);     // never 0
            best = key > best ? key : best;
          }
        const uint64_t m = wave_max_u64(best);
        if (m != 0) {
          const int i = (int)(0xFFFFFFFFu - (uint32_t)m);
          if (i % kRouteThreads == tid) done_mask |= 1ull << (i / kRouteThreads);
        }
        if (lane == 0) s_wtop[wid][r] = m;
      }
      __syncthreads();
      if (wid == 0) {
        uint64_t c[kRouteThreads / 64];
#pragma unroll
        for (int w = 0; w < kRouteThreads / 64; ++w) c[w] = (lane < nT) ? s_wtop[w][lane] : 0ull;
        for (int r = 0; r < nT; ++r) {
          uint64_t best = 0;
#pragma unroll
          for (int w = 0; w < kRouteThreads / 64; ++w) best = c[w] > best ? c[w] : best;
          const uint64_t m = wave_max_u64(best);
#pragma unroll
          for (int w = 0; w < kRouteThreads / 64; ++w) if (c[w] == m) c[w] = 0;
          if (lane == 0) s_chunks[r] = c_lo + (int)(0xFFFFFFFFu - (uint32_t)m);
        }
      }
    }
    __syncthreads();
    // chosen chunks in ascending order
    if (tid < nT) {
      const int c = s_chunks[tid];
      int rank = 0;
      for (int j = 0; j < nT; ++j) rank += (s_chunks[j] < c);
      s_sorted[rank] = c;
    }
    __syncthreads();
    // level 2: score every group of every chosen chunk
    for (int i = tid; i < nT * gpc; i += kRouteThreads)
      s_rowmap[i] = (int)(kvg * a.n_gs_cap + (int64_t)s_sorted[i / gpc] * gpc + (i % gpc));
    __syncthreads();
    score_rows<T, D>(a.group_sum, 0, nT * gpc, qv, dyn, s_rowmap);
    __syncthreads();
    if (tid < nT) {
      // top TG of this chunk's gpc groups, then ascending
      uint64_t picked_mask = 0;
      for (int r = 0; r < TG; ++r) {
        uint64_t best = 0;
        int bj = 0;
        for (int j = 0; j < gpc; ++j) {
          if ((picked_mask >> j) & 1ull) continue;
          const uint64_t k = score_key(dyn[tid * gpc + j], j);
          if (k > best) { best = k; bj = j; }
        }
        picked_mask |= 1ull << bj;
      }
      int o = 0;
      for (int j = 0; j < gpc; ++j)
        if ((picked_mask >> j) & 1ull) s_groups[tid * TG + (o++)] = s_sorted[tid] * gpc + j;
    }
    __syncthreads();
  }

  // assemble the ascending token list
  const int sinks_end = min(c_lo, kappa) * C;                // [0, sinks_end)
  const int n_routed = max(nT, 0) * TG * GR;
  const int loc_lo = max(c_lo, kappa - a.local_chunks);      // local chunks [loc_lo, kappa)
  const int n_local = max(0, kappa - loc_lo) * C;
  const int cur0 = kappa * C;
  const int o_routed = sinks_end, o_local = o_routed + n_routed, o_cur = o_local + n_local;
  // prefill lists stop before the block: its queries add their own keys
  const int n_cur = a.prefill ? 0 : (n - cur0);
  const int total = o_cur + n_cur;
  int32_t* out = a.prefill ? a.blk_idx + ((int64_t)bg * a.nblk + blk) * a.K : a.sel_idx + bg * a.n_cap;
  for (int i = tid; i < sinks_end; i += kRouteThreads) out[i] = i;
  for (int i = tid; i < n_routed; i += kRouteThreads) out[o_routed + i] = s_groups[i / GR] * GR + (i % GR);
  for (int i = tid; i < n_local; i += kRouteThreads) out[o_local + i] = loc_lo * C + i;
  for (int i = tid; i < n_cur; i += kRouteThreads) out[o_cur + i] = cur0 + i;
  if (tid == 0) {
    if (a.prefill) a.blk_count[bg * a.nblk + blk] = total;
    else a.sel_count[bg] = total;
  }
}

hipError_t launch_route(const RouteArgs& a, int dtype, int d, hipStream_t s) {
  if (a.groups.n == 0) return hipSuccess;
  const int gpc = a.chunk / a.group;
  if (a.top_chunks * a.top_groups > kMaxRoutedGroups || a.top_chunks > 64 || gpc > 64)
    return hipErrorInvalidValue;
  const int ncand_max = a.n / a.chunk + 1;
  if (ncand_max > 16384) return hipErrorInvalidValue;
  const size_t dyn = 4 * (size_t)std::max(ncand_max, a.top_chunks * gpc);
  if (a.prefill && (d > 128 || a.nblk < 1)) return hipErrorInvalidValue;
  dim3 grid(a.prefill ? a.nblk : 1, a.groups.n, a.B), block(kRouteThreads);
  if (dtype == 0 && d == 128) hipLaunchKernelGGL((route_kernel<bf16_t, 128>), grid, block, dyn, s, a);
  else if (dtype == 0 && d == 64) hipLaunchKernelGGL((route_kernel<bf16_t, 64>), grid, block, dyn, s, a);
  else if (dtype == 1 && d == 128) hipLaunchKernelGGL((route_kernel<float, 128>), grid, block, dyn, s, a);
  else if (dtype == 1 && d == 64) hipLaunchKernelGGL((route_kernel<float, 64>), grid, block, dyn, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sa
