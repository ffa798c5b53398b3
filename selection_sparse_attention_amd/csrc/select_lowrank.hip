// Top-p / top-k token selector over the low-rank index ("Full Attention
// Strikes Back" summary, Methodology items 2, 3 and 5; AoH summary,
// Methodology item 4 for the GQA group mean).
//
// For every (sequence b, retrieval group g) row:
//   qbar = mean_h q_idx[b,h]  over the group's query heads
//   l_j  = qbar . k_idx[b,g,j] / 4        (1/sqrt(r), r = 16)
//   rank = (l desc, j asc); keep the shortest prefix whose softmax mass is
//          >= p (top-p; raised to min_tokens), or the first k (top-k).
//
// The cut is found without sorting (the summary describes a sort-free,
// histogram-based threshold): logits are mapped to order-preserving 32-bit
// keys and resolved by three radix levels (12 + 12 + 8 bits).  Each level is
// one launch over the row's tiles; every tile builds an LDS histogram of
// counts and fp64 masses, merges it into the row's global histogram with
// atomics, and the last tile to finish scans the merged histogram for the
// bucket that holds the cut.  The first level also computes and stores the
// logits (4 B/token), so only the scan reads the 32 B/token index.  Masses at
// level 1 are taken relative to each bucket's upper bound (a data-independent
// reference, so per-tile histograms add without knowing the max); later
// levels use the top bucket's bound R.  Ties at the final key go to the lowest
// positions; a decoupled look-back scan over the tiles then writes the
// selected positions in ascending order.
#include "args.hpp"
#include "common.hpp"

namespace sa {

constexpr int kTile = 1024;        // tokens per workgroup
constexpr int kThreads = 256;
constexpr int kPer = kTile / kThreads;
constexpr int kSpinLimit = 1 << 24;

enum : int { CRIT_MASS = 1, CRIT_COUNT = 2 };

__device__ __forceinline__ void row_coords(const SelectArgs& a, int row, int& b, int& g) {
  b = row / a.groups.n;
  g = a.groups.ids[row % a.groups.n];
}

// Upper bound (as a double) of the values whose key has the given top bits.
__device__ __forceinline__ double bucket_hi(uint32_t b, int shift) {
  const uint32_t top = (b << shift) | ((shift == 0) ? 0u : ((1u << shift) - 1u));
  return (double)key_to_float(top);
}

// ------------------------------------------------------------------ clear
// Zero the per-row histograms, counters and look-back words; set the row
// state.  One workgroup per row.
__global__ __launch_bounds__(kThreads) void select_clear_kernel(SelectArgs a) {
  const int row = blockIdx.x;
  for (int i = threadIdx.x; i < 4096; i += kThreads) {
    a.cnt1[(int64_t)row * 4096 + i] = 0; a.mass1[(int64_t)row * 4096 + i] = 0.0;
    a.cnt2[(int64_t)row * 4096 + i] = 0; a.mass2[(int64_t)row * 4096 + i] = 0.0;
  }
  for (int i = threadIdx.x; i < 256; i += kThreads) {
    a.cnt3[(int64_t)row * 256 + i] = 0; a.mass3[(int64_t)row * 256 + i] = 0.0;
  }
  for (int i = threadIdx.x; i < a.tiles; i += kThreads) a.lookback[(int64_t)row * a.tiles + i] = 0;
  if (threadIdx.x < 4) a.done[row * 4 + threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    RowState st{};
    st.target_count = a.target_count;
    st.crit = (a.use_mass ? CRIT_MASS : 0) | (a.target_count > 0 ? CRIT_COUNT : 0);
    st.all = a.select_all;
    st.m = a.select_all ? a.n : 0;
    a.state[row] = st;
  }
}

// ------------------------------------------------------------------ find
// Run by the last workgroup of a level.  Scans NB buckets from the highest
// key down, finds the bucket holding the cut under the live criteria, and
// folds everything above it into the row state.
template <int NB, int LEVEL>
__device__ void find_cut(const SelectArgs& a, int row, const uint32_t* gcnt, const double* gmass,
                         bool mass, uint32_t* s_c, double* s_w) {
  // s_c / s_w: the caller's LDS histogram arrays, reused as scratch (s_w is
  // only touched when masses are tracked)
  constexpr int PER = NB / kThreads;           // buckets per thread (16 or 1)
  __shared__ double s_scan_d[kThreads / 64];
  __shared__ int64_t s_scan_i[kThreads / 64];
  __shared__ int s_top;
  __shared__ int s_bm, s_bc;
  RowState& st = a.state[row];
  const int tid = threadIdx.x;

  __syncthreads();
  for (int i = tid; i < NB; i += kThreads) {
    s_c[i] = ld_agent(gcnt + i);
    if (mass) s_w[i] = ld_agent(gmass + i);
  }
  if (tid == 0) { s_top = -1; s_bm = -1; s_bc = -1; }
  __syncthreads();
  if (LEVEL == 1 && mass) {
    // reference R = upper bound of the highest non-empty bucket
    for (int i = tid; i < NB; i += kThreads) if (s_c[i]) atomicMax(&s_top, i);
    __syncthreads();
    const double R = bucket_hi((uint32_t)s_top, 20);
    for (int i = tid; i < NB; i += kThreads)
      if (s_c[i]) s_w[i] = s_w[i] * exp(bucket_hi((uint32_t)i, 20) - R);
    if (tid == 0) st.R = R;
    __syncthreads();
  }
  // thread t owns buckets NB-1-PER*t ... NB-PER*t (descending key order)
  double tw = 0.0; int64_t tc = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int bk = NB - 1 - (PER * tid + k);
    if (mass) tw += s_w[bk];
    tc += s_c[bk];
  }
  double totw; int64_t totc;
  const double pre_w = block_exclusive_scan<double, kThreads>(tw, s_scan_d, &totw);
  const int64_t pre_c = block_exclusive_scan<int64_t, kThreads>(tc, s_scan_i, &totc);
  const int crit = st.crit;
  if (LEVEL == 1 && mass && tid == 0) st.target_mass = totw * a.top_p;
  __syncthreads();
  const double tmass = (LEVEL == 1 && mass) ? totw * a.top_p : st.target_mass;
  const double base_w = st.mass_above;
  const int64_t base_c = st.count_above;
  {
    double cw = base_w + pre_w; int64_t cc = base_c + pre_c;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int bk = NB - 1 - (PER * tid + k);
      const double nw = cw + (mass ? s_w[bk] : 0.0);
      const int64_t nc = cc + s_c[bk];
      if ((crit & CRIT_MASS) && s_c[bk] && cw < tmass && nw >= tmass) s_bm = bk;
      if ((crit & CRIT_COUNT) && s_c[bk] && cc < st.target_count && nc >= st.target_count) s_bc = bk;
      cw = nw; cc = nc;
    }
  }
  __syncthreads();
  if (tid != 0) return;
  const bool m_on = (crit & CRIT_MASS) != 0, c_on = (crit & CRIT_COUNT) != 0;
  int bm = s_bm, bc = s_bc;
  if (m_on && bm < 0 && LEVEL > 1) {
    // The previous level placed the crossing inside this prefix; a last-place
    // disagreement between the two levels' mass sums lands it on the first or
    // last non-empty bucket.
    int hi_b = -1, lo_b = -1;
    for (int bk = NB - 1; bk >= 0; --bk)
      if (s_c[bk]) { if (hi_b < 0) hi_b = bk; lo_b = bk; }
    bm = (base_w >= tmass) ? hi_b : lo_b;
  }
  // m_on: the mass crossing decides unless the count crossing lies further
  // down the order (a lower bucket); both stay live while they share a bucket
  int bstar, ncrit;
  if (m_on && c_on) {
    const bool mass_wins = (bc < 0) || (bm >= 0 && bm < bc);
    const bool count_wins = (bm >= 0) && (bc >= 0) && (bc < bm);
    bstar = count_wins ? bc : bm;
    ncrit = mass_wins ? CRIT_MASS : (count_wins ? CRIT_COUNT : (CRIT_MASS | CRIT_COUNT));
  } else {
    bstar = m_on ? bm : bc;
    ncrit = crit;
  }
  if (bstar < 0) {                 // the target lies past the last token
    st.all = 1;
    st.m = a.n;
    return;
  }
  double aw = 0.0;
  int64_t ac = 0;
  for (int bk = NB - 1; bk > bstar; --bk) {
    if (mass) aw += s_w[bk];
    ac += s_c[bk];
  }
  const double above_w = base_w + aw;
  const int64_t above_c = base_c + ac;
  constexpr int BITS = (NB == 4096) ? 12 : 8;
  const uint32_t prefix = (LEVEL == 1) ? (uint32_t)bstar : ((st.prefix << BITS) | (uint32_t)bstar);
  st.mass_above = above_w;
  st.count_above = above_c;
  st.crit = ncrit;
  st.prefix = prefix;
  if (LEVEL == 3) {
    const int64_t ties = s_c[bstar];
    int64_t need = 1;
    if (ncrit & CRIT_MASS) {
      const double e = exp((double)key_to_float(prefix) - st.R);
      const double c = ceil((tmass - above_w) / e);
      need = (c >= (double)ties) ? ties : (c <= 1.0 ? 1 : (int64_t)c);
    }
    if (ncrit & CRIT_COUNT) {
      const int64_t nc = (int64_t)st.target_count - above_c;
      need = need > nc ? need : nc;
    }
    if (need > ties) need = ties;
    if (need < 1) need = 1;
    st.cut_key = prefix;
    st.need = (int32_t)need;
    st.m = (int32_t)(above_c + need);
  }
}

// Merge a tile's LDS histogram into the row histogram; the last tile of the
// row runs find_cut.  Returns nothing; side effects only.
template <int NB, int LEVEL>
__device__ void merge_and_find(const SelectArgs& a, int row, uint32_t* lc, double* lw,
                               uint32_t* gcnt, double* gmass, bool mass) {
  __shared__ int s_last;
  for (int i = threadIdx.x; i < NB; i += kThreads) {
    if (lc[i]) {
      atomicAdd(gcnt + i, lc[i]);
      if (mass) unsafeAtomicAdd(gmass + i, lw[i]);
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = atomicAdd(&a.done[row * 4 + LEVEL], 1u);
    s_last = (t == (uint32_t)a.tiles - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  find_cut<NB, LEVEL>(a, row, gcnt, gmass, mass, lc, lw);
}

__device__ __forceinline__ bool row_active(const RowState& st) { return !st.all; }

// ------------------------------------------------------------------ level 1
// Logits of one tile (written to the workspace) and their 12-bit histogram.
template <typename T, bool MASS>
__global__ __launch_bounds__(kThreads) void select_scan_kernel(SelectArgs a) {
  __shared__ uint32_t lc[4096];
  __shared__ double lw[MASS ? 4096 : 1];
  const int row = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  int b, g;
  row_coords(a, row, b, g);
  if (a.select_all) return;
  for (int i = tid; i < 4096; i += kThreads) { lc[i] = 0; if (MASS) lw[i] = 0.0; }

  // qbar: mean of the group's index queries (exact for power-of-two G on
  // lattice inputs)
  float qb[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) qb[c] = 0.f;
  for (int hh = 0; hh < a.G; ++hh) {
    const float* qp = a.q_idx + ((int64_t)b * a.Hq + g * a.G + hh) * 16;
#pragma unroll
    for (int c = 0; c < 16; ++c) qb[c] += qp[c];
  }
  const float invG = 1.0f / (float)a.G;
#pragma unroll
  for (int c = 0; c < 16; ++c) qb[c] *= invG;
  __syncthreads();

  const int64_t krow = ((int64_t)b * a.Hkv + g) * a.n_cap;
  float* lg = a.logits + (int64_t)row * a.row_stride;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = tile * kTile + i * kThreads + tid;
    if (j < a.n) {
      float kv[16];
      VecLoad<T, 16>::run(a.k_idx, (krow + j) * 16, kv);
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) acc = fmaf(qb[c], kv[c], acc);
      float l = acc * 0.25f;
      if (l == 0.f) l = 0.f;                       // fold -0 into +0
      lg[j] = l;
      const uint32_t key = order_key(l);
      const uint32_t bk = key >> 20;
      atomicAdd(&lc[bk], 1u);
      if (MASS) atomicAdd(&lw[bk], exp((double)l - bucket_hi(bk, 20)));
    }
  }
  __syncthreads();
  merge_and_find<4096, 1>(a, row, lc, MASS ? lw : nullptr, a.cnt1 + (int64_t)row * 4096,
                          a.mass1 + (int64_t)row * 4096, MASS);
}

// ------------------------------------------------------------------ levels 2, 3
template <int LEVEL, bool MASS>
__global__ __launch_bounds__(kThreads) void select_level_kernel(SelectArgs a) {
  constexpr int NB = (LEVEL == 2) ? 4096 : 256;
  constexpr int SHIFT = (LEVEL == 2) ? 8 : 0;
  constexpr int PSHIFT = (LEVEL == 2) ? 20 : 8;
  __shared__ uint32_t lc[NB];
  __shared__ double lw[MASS ? NB : 1];
  const int row = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  const RowState st = a.state[row];
  if (!row_active(st)) return;
  for (int i = tid; i < NB; i += kThreads) { lc[i] = 0; if (MASS) lw[i] = 0.0; }
  __syncthreads();
  const float* lg = a.logits + (int64_t)row * a.row_stride;
  const double R = st.R;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = tile * kTile + i * kThreads + tid;
    if (j < a.n) {
      const float l = lg[j];
      const uint32_t key = order_key(l);
      if ((key >> PSHIFT) == st.prefix) {
        const uint32_t bk = (key >> SHIFT) & (NB - 1);
        atomicAdd(&lc[bk], 1u);
        if (MASS) atomicAdd(&lw[bk], exp((double)l - R));
      }
    }
  }
  __syncthreads();
  uint32_t* gc = (LEVEL == 2 ? a.cnt2 + (int64_t)row * 4096 : a.cnt3 + (int64_t)row * 256);
  double* gw = (LEVEL == 2 ? a.mass2 + (int64_t)row * 4096 : a.mass3 + (int64_t)row * 256);
  merge_and_find<NB, LEVEL>(a, row, lc, MASS ? lw : nullptr, gc, gw, MASS);
}

// ------------------------------------------------------------------ compact
// Writes the selected positions of a row in ascending order.  Tiles publish
// (strict, tie) counts and look back over earlier tiles for their prefix.
constexpr uint64_t kFlagAgg = 1ull << 62, kFlagIncl = 2ull << 62;
__device__ __forceinline__ uint64_t pack_counts(uint64_t flag, uint32_t s, uint32_t t) {
  return flag | ((uint64_t)s << 31) | (uint64_t)t;
}

__global__ __launch_bounds__(kThreads) void select_compact_kernel(SelectArgs a) {
  __shared__ uint32_t s_scan[kThreads / 64];
  __shared__ uint32_t s_pre_s, s_pre_t;
  const int row = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  int b, g;
  row_coords(a, row, b, g);
  const RowState st = a.state[row];
  const int64_t orow = ((int64_t)b * a.Hkv + g) * a.n_cap;
  const float* lg = a.logits + (int64_t)row * a.row_stride;
  const int j0 = tile * kTile + tid * kPer;   // this thread's 4 consecutive tokens

  uint32_t strict_f = 0, tie_f = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = j0 + i;
    if (j >= a.n) continue;
    if (st.all) { strict_f |= 1u << i; continue; }
    const uint32_t key = order_key(lg[j]);
    if (key > st.cut_key) strict_f |= 1u << i;
    else if (key == st.cut_key) tie_f |= 1u << i;
  }
  uint32_t tot_s, tot_t;
  const uint32_t ex_s = block_exclusive_scan<uint32_t, kThreads>(__popc(strict_f), s_scan, &tot_s);
  const uint32_t ex_t = block_exclusive_scan<uint32_t, kThreads>(__popc(tie_f), s_scan, &tot_t);

  if (tid == 0) {
    uint64_t* lb = a.lookback + (int64_t)row * a.tiles;
    uint32_t ps = 0, pt = 0;
    if (tile == 0) {
      st_agent(lb, pack_counts(kFlagIncl, tot_s, tot_t));
    } else {
      st_agent(lb + tile, pack_counts(kFlagAgg, tot_s, tot_t));
      int p = tile - 1;
      int spins = 0;
      while (p >= 0) {
        const uint64_t w = ld_agent(lb + p);
        const uint64_t f = w & (3ull << 62);
        if (f == 0) {
          if (++spins > kSpinLimit) { a.state[row].err = 1; break; }
          continue;
        }
        ps += (uint32_t)((w >> 31) & 0x7FFFFFFFu);
        pt += (uint32_t)(w & 0x7FFFFFFFu);
        if (f == kFlagIncl) break;
        --p;
      }
      st_agent(lb + tile, pack_counts(kFlagIncl, ps + tot_s, pt + tot_t));
    }
    s_pre_s = ps; s_pre_t = pt;
    if (tile == a.tiles - 1) a.sel_count[(int64_t)b * a.Hkv + g] = st.m;
  }
  __syncthreads();
  const uint32_t need = st.all ? 0u : (uint32_t)st.need;
  uint32_t s_before = s_pre_s + ex_s, t_before = s_pre_t + ex_t;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = j0 + i;
    if (strict_f & (1u << i)) {
      const uint32_t o = s_before + (t_before < need ? t_before : need);
      a.sel_idx[orow + o] = j;
      ++s_before;
    } else if (tie_f & (1u << i)) {
      if (t_before < need) a.sel_idx[orow + s_before + t_before] = j;
      ++t_before;
    }
  }
}

template <typename T>
static hipError_t run_select(const SelectArgs& a, hipStream_t s) {
  const int rows = a.B * a.groups.n;
  dim3 grid(a.tiles, rows);
  hipLaunchKernelGGL(select_clear_kernel, dim3(rows), dim3(kThreads), 0, s, a);
  if (!a.select_all) {
    if (a.use_mass) {
      hipLaunchKernelGGL((select_scan_kernel<T, true>), grid, dim3(kThreads), 0, s, a);
      hipLaunchKernelGGL((select_level_kernel<2, true>), grid, dim3(kThreads), 0, s, a);
      hipLaunchKernelGGL((select_level_kernel<3, true>), grid, dim3(kThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL((select_scan_kernel<T, false>), grid, dim3(kThreads), 0, s, a);
      hipLaunchKernelGGL((select_level_kernel<2, false>), grid, dim3(kThreads), 0, s, a);
      hipLaunchKernelGGL((select_level_kernel<3, false>), grid, dim3(kThreads), 0, s, a);
    }
  }
  hipLaunchKernelGGL(select_compact_kernel, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select_lowrank(const SelectArgs& a, int dtype, hipStream_t s) {
  if (a.B * a.groups.n == 0) return hipSuccess;
  return dtype == 0 ? run_select<bf16_t>(a, s) : run_select<float>(a, s);
}

}  // namespace sa
