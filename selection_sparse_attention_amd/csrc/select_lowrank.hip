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
// keys and resolved by three radix levels (12 + 12 + 8 bits).
//
//   scan   (tiles x rows)  logits to the workspace (4 B/token) + level-1
//                          histogram of counts and fp64 masses
//   find1  (rows)          cut bucket of level 1
//   level2 (tiles x rows)  histogram of the next 12 bits inside the cut bucket
//   find2  (rows)
//   level3 (tiles x rows)  the last 8 bits
//   find3  (rows)          exact cut key and how many of its ties to keep
//   compact(tiles x rows)  ascending positions, via a decoupled look-back
//
// Tiles merge their LDS histograms into the row's histogram with atomics; the
// per-row find kernels read them after the kernel boundary, so no tile ever
// waits on another (an agent-scope fence would write back the die's L2).  Only
// the scan reads the 32 B/token index.  Level-1 masses are taken relative to
// each bucket's upper bound - a data-independent reference, so tile
// histograms add without knowing the maximum - and rescaled to the top
// bucket's bound R when merged; later levels use R directly.  Every find
// kernel zeroes the histogram it consumed and the scan zeroes the look-back
// words, so a workspace that starts zero-filled stays reusable.
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

// Add a tile's LDS histogram into the row's histogram (non-empty buckets).
template <int NB>
__device__ __forceinline__ void merge_hist(const uint32_t* lc, const double* lw, uint32_t* gc,
                                           double* gw, bool mass) {
  for (int i = threadIdx.x; i < NB; i += kThreads) {
    const uint32_t c = lc[i];
    if (c) {
      atomicAdd(gc + i, c);
      if (mass) unsafeAtomicAdd(gw + i, lw[i]);
    }
  }
}

// ------------------------------------------------------------------ scan
template <typename T, bool MASS>
__global__ __launch_bounds__(kThreads) void select_scan_kernel(SelectArgs a) {
  __shared__ uint32_t lc[4096];
  __shared__ double lw[MASS ? 4096 : 1];
  const int row = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  int b, g;
  row_coords(a, row, b, g);
  for (int i = tid; i < 4096; i += kThreads) { lc[i] = 0; if (MASS) lw[i] = 0.0; }
  if (tid == 0) a.lookback[(int64_t)row * a.tiles + tile] = 0;

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
  float kv[kPer][16];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {                 // all loads in flight first
    const int j = tile * kTile + i * kThreads + tid;
    if (j < a.n) VecLoad<T, 16>::run(a.k_idx, (krow + j) * 16, kv[i]);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = tile * kTile + i * kThreads + tid;
    if (j < a.n) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c) acc = fmaf(qb[c], kv[i][c], acc);
      float l = acc * 0.25f;
      if (l == 0.f) l = 0.f;                       // fold -0 into +0
      lg[j] = l;
      const uint32_t bk = order_key(l) >> 20;
      atomicAdd(&lc[bk], 1u);
      if (MASS) atomicAdd(&lw[bk], exp((double)l - bucket_hi(bk, 20)));
    }
  }
  __syncthreads();
  merge_hist<4096>(lc, lw, a.cnt1 + (int64_t)row * 4096, a.mass1 + (int64_t)row * 4096, MASS);
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
  if (st.all) return;
  for (int i = tid; i < NB; i += kThreads) { lc[i] = 0; if (MASS) lw[i] = 0.0; }
  __syncthreads();
  const float* lg = a.logits + (int64_t)row * a.row_stride;
  float lv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = tile * kTile + i * kThreads + tid;
    lv[i] = (j < a.n) ? lg[j] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = tile * kTile + i * kThreads + tid;
    if (j < a.n) {
      const uint32_t key = order_key(lv[i]);
      if ((key >> PSHIFT) == st.prefix) {
        const uint32_t bk = (key >> SHIFT) & (NB - 1);
        atomicAdd(&lc[bk], 1u);
        if (MASS) atomicAdd(&lw[bk], exp((double)lv[i] - st.R));
      }
    }
  }
  __syncthreads();
  if (LEVEL == 2)
    merge_hist<NB>(lc, lw, a.cnt2 + (int64_t)row * 4096, a.mass2 + (int64_t)row * 4096, MASS);
  else
    merge_hist<NB>(lc, lw, a.cnt3 + (int64_t)row * 256, a.mass3 + (int64_t)row * 256, MASS);
}

// ------------------------------------------------------------------ find
// One workgroup per row.  Scans the row's histogram of this level from the
// highest key down, finds the bucket that holds the cut under the live
// criteria, folds every bucket above it into the row state, and zeroes the
// histogram for the next call.
template <int LEVEL, bool MASS>
__global__ __launch_bounds__(kThreads) void select_find_kernel(SelectArgs a) {
  constexpr int NB = (LEVEL == 3) ? 256 : 4096;
  constexpr int PER = NB / kThreads;               // buckets per thread (16 or 1)
  constexpr int BITS = (NB == 4096) ? 12 : 8;
  __shared__ uint32_t s_c[NB];
  __shared__ double s_w[MASS ? NB : 1];
  __shared__ double s_scan_d[kThreads / 64];
  __shared__ int64_t s_scan_i[kThreads / 64];
  __shared__ int s_top, s_bm, s_bc;
  __shared__ double s_bm_w, s_bc_w;          // mass above the crossing buckets
  __shared__ int64_t s_bm_c, s_bc_c;         // count above the crossing buckets
  const int row = blockIdx.x, tid = threadIdx.x;
  RowState& st = a.state[row];
  uint32_t* gc = (LEVEL == 1 ? a.cnt1 + (int64_t)row * 4096
                             : LEVEL == 2 ? a.cnt2 + (int64_t)row * 4096 : a.cnt3 + (int64_t)row * 256);
  double* gw = (LEVEL == 1 ? a.mass1 + (int64_t)row * 4096
                           : LEVEL == 2 ? a.mass2 + (int64_t)row * 4096 : a.mass3 + (int64_t)row * 256);

  if (LEVEL == 1) {
    if (tid == 0) {
      RowState init{};
      init.target_count = a.target_count;
      init.crit = (MASS ? CRIT_MASS : 0) | (a.target_count > 0 ? CRIT_COUNT : 0);
      st = init;
    }
    __syncthreads();
  } else {
    if (st.all) return;
  }
  {
    // every load in flight before the zeroing stores (they alias the loads)
    uint32_t cv[PER];
    double wv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      cv[k] = gc[tid + k * kThreads];
      wv[k] = MASS ? gw[tid + k * kThreads] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      s_c[tid + k * kThreads] = cv[k];
      if (MASS) s_w[tid + k * kThreads] = wv[k];
      gc[tid + k * kThreads] = 0;
      if (MASS) gw[tid + k * kThreads] = 0.0;
    }
  }
  if (tid == 0) { s_top = -1; s_bm = -1; s_bc = -1; }
  __syncthreads();
  if (LEVEL == 1 && MASS) {
    // reference R = upper bound of the highest non-empty bucket
    for (int i = tid; i < NB; i += kThreads) if (s_c[i]) atomicMax(&s_top, i);
    __syncthreads();
    const double R = bucket_hi((uint32_t)max(s_top, 0), 20);
    for (int i = tid; i < NB; i += kThreads)
      if (s_c[i]) s_w[i] = s_w[i] * exp(bucket_hi((uint32_t)i, 20) - R);
    if (tid == 0) st.R = R;
    __syncthreads();
  }
  // thread t owns buckets NB-1-PER*t ... NB-PER*t (descending key order)
  double tw = 0.0;
  int64_t tc = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int bk = NB - 1 - (PER * tid + k);
    if (MASS) tw += s_w[bk];
    tc += s_c[bk];
  }
  double totw;
  int64_t totc;
  const double pre_w = block_exclusive_scan<double, kThreads>(tw, s_scan_d, &totw);
  const int64_t pre_c = block_exclusive_scan<int64_t, kThreads>(tc, s_scan_i, &totc);
  const int crit = st.crit;
  const double tmass = (LEVEL == 1) ? totw * a.top_p : st.target_mass;
  const double base_w = (LEVEL == 1) ? 0.0 : st.mass_above;
  const int64_t base_c = (LEVEL == 1) ? 0 : st.count_above;
  const int64_t tcount = st.target_count;
  {
    double cw = base_w + pre_w;
    int64_t cc = base_c + pre_c;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int bk = NB - 1 - (PER * tid + k);
      const double nw = cw + (MASS ? s_w[bk] : 0.0);
      const int64_t nc = cc + s_c[bk];
      if ((crit & CRIT_MASS) && s_c[bk] && cw < tmass && nw >= tmass) {
        s_bm = bk; s_bm_w = cw; s_bm_c = cc;
      }
      if ((crit & CRIT_COUNT) && s_c[bk] && cc < tcount && nc >= tcount) {
        s_bc = bk; s_bc_w = cw; s_bc_c = cc;
      }
      cw = nw;
      cc = nc;
    }
  }
  __syncthreads();
  if (tid != 0) return;
  if (LEVEL == 1) st.target_mass = tmass;
  const bool m_on = (crit & CRIT_MASS) != 0, c_on = (crit & CRIT_COUNT) != 0;
  int bm = s_bm, bc = s_bc;
  double bm_w = s_bm_w;
  int64_t bm_c = s_bm_c;
  if (m_on && bm < 0 && LEVEL > 1) {
    // The previous level placed the crossing inside this prefix; a last-place
    // disagreement between the two levels' mass sums lands it on the first or
    // last non-empty bucket (rare: a serial walk is fine here).
    int hi_b = -1, lo_b = -1;
    for (int bk = NB - 1; bk >= 0; --bk)
      if (s_c[bk]) { if (hi_b < 0) hi_b = bk; lo_b = bk; }
    bm = (base_w >= tmass) ? hi_b : lo_b;
    bm_w = base_w;
    bm_c = base_c;
    for (int bk = NB - 1; bk > bm && bm >= 0; --bk) { if (MASS) bm_w += s_w[bk]; bm_c += s_c[bk]; }
  }
  // the mass crossing decides unless the count crossing lies further down the
  // order (a lower bucket); both stay live while they share a bucket
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
  // everything above the chosen bucket, as accumulated by the scan
  const bool from_mass = (bstar == bm) && m_on;
  const double above_w = from_mass ? bm_w : s_bc_w;
  const int64_t above_c = from_mass ? bm_c : s_bc_c;
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
      const int64_t nc = tcount - above_c;
      need = need > nc ? need : nc;
    }
    if (need > ties) need = ties;
    if (need < 1) need = 1;
    st.cut_key = prefix;
    st.need = (int32_t)need;
    st.m = (int32_t)(above_c + need);
  }
}

// ------------------------------------------------------------------ compact
// Writes the selected positions of a row in ascending order.  Tiles publish
// (strict, tie) counts and look back over earlier tiles for their prefix; the
// counts travel inside the 64-bit flag words, so relaxed atomics suffice.
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
  const int64_t orow = ((int64_t)b * a.Hkv + g) * a.n_cap;
  const int j0 = tile * kTile + tid * kPer;   // this thread's 4 consecutive tokens
  const bool all = a.select_all || a.state[row].all;
  if (all) {                                   // every token: position j goes to slot j
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (j0 + i < a.n) a.sel_idx[orow + j0 + i] = j0 + i;
    if (tile == 0 && tid == 0) a.sel_count[(int64_t)b * a.Hkv + g] = a.n;
    return;
  }
  const RowState st = a.state[row];
  const float* lg = a.logits + (int64_t)row * a.row_stride;
  uint32_t strict_f = 0, tie_f = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = j0 + i;
    if (j >= a.n) continue;
    const uint32_t key = order_key(lg[j]);
    if (key > st.cut_key) strict_f |= 1u << i;
    else if (key == st.cut_key) tie_f |= 1u << i;
  }
  uint32_t tot_s, tot_t;
  const uint32_t ex_s = block_exclusive_scan<uint32_t, kThreads>(__popc(strict_f), s_scan, &tot_s);
  const uint32_t ex_t = block_exclusive_scan<uint32_t, kThreads>(__popc(tie_f), s_scan, &tot_t);

  if (tid < 64) {
    // wave 0 looks back over up to 64 predecessors at once: lane i reads tile
    // (base - i); the window is consumed up to the nearest inclusive prefix
    uint64_t* lb = a.lookback + (int64_t)row * a.tiles;
    const int lane = tid;
    uint32_t ps = 0, pt = 0;
    if (tile == 0) {
      if (lane == 0) st_agent(lb, pack_counts(kFlagIncl, tot_s, tot_t));
    } else {
      if (lane == 0) st_agent(lb + tile, pack_counts(kFlagAgg, tot_s, tot_t));
      int base = tile - 1;
      int spins = 0;
      while (base >= 0) {
        const int p = base - lane;
        uint64_t w = (p >= 0) ? ld_agent(lb + p) : kFlagIncl;   // before tile 0: an empty prefix
        const uint64_t f = w & (3ull << 62);
        // all lanes up to the first inclusive one must have published
        const uint64_t incl_mask = __ballot(f == kFlagIncl);
        const int first_incl = incl_mask ? __ffsll((unsigned long long)incl_mask) - 1 : 64;
        const uint64_t ready = __ballot(f != 0);
        const int need_lanes = (first_incl < 64) ? first_incl + 1 : 64;
        const uint64_t want = (need_lanes == 64) ? ~0ull : ((1ull << need_lanes) - 1);
        if ((ready & want) != want) {
          if (++spins > kSpinLimit) { if (lane == 0) a.state[row].err = 1; break; }
          continue;
        }
        uint32_t vs = (lane < need_lanes && p >= 0) ? (uint32_t)((w >> 31) & 0x7FFFFFFFu) : 0u;
        uint32_t vt = (lane < need_lanes && p >= 0) ? (uint32_t)(w & 0x7FFFFFFFu) : 0u;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) { vs += __shfl_xor(vs, o); vt += __shfl_xor(vt, o); }
        ps += vs;
        pt += vt;
        if (first_incl < 64) break;
        base -= 64;
      }
      if (lane == 0) st_agent(lb + tile, pack_counts(kFlagIncl, ps + tot_s, pt + tot_t));
    }
    if (lane == 0) {
      s_pre_s = ps;
      s_pre_t = pt;
      if (tile == a.tiles - 1) a.sel_count[(int64_t)b * a.Hkv + g] = st.m;
    }
  }
  __syncthreads();
  const uint32_t need = (uint32_t)st.need;
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

template <typename T, bool MASS>
static void run_levels(const SelectArgs& a, hipStream_t s) {
  const int rows = a.B * a.groups.n;
  dim3 grid(a.tiles, rows);
  hipLaunchKernelGGL((select_scan_kernel<T, MASS>), grid, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((select_find_kernel<1, MASS>), dim3(rows), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((select_level_kernel<2, MASS>), grid, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((select_find_kernel<2, MASS>), dim3(rows), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((select_level_kernel<3, MASS>), grid, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL((select_find_kernel<3, MASS>), dim3(rows), dim3(kThreads), 0, s, a);
}

hipError_t launch_select_lowrank(const SelectArgs& a, int dtype, hipStream_t s) {
  const int rows = a.B * a.groups.n;
  if (rows == 0) return hipSuccess;
  if (!a.select_all) {
    if (dtype == 0) {
      if (a.use_mass) run_levels<bf16_t, true>(a, s); else run_levels<bf16_t, false>(a, s);
    } else {
      if (a.use_mass) run_levels<float, true>(a, s); else run_levels<float, false>(a, s);
    }
  }
  hipLaunchKernelGGL(select_compact_kernel, dim3(a.tiles, rows), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
