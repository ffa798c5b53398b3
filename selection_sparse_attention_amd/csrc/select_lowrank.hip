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
//   scan (tiles x rows)  logits to the workspace (4 B/token) + level-1
//                        histogram of counts and fp64 masses, merged into the
//                        row's histogram with atomics
//   row  (rows)          one 1024-thread workgroup per row: the level-1 cut,
//                        then the logits of the cut bucket gathered into LDS
//                        and levels 2 and 3 over them (LDS histograms): the
//                        exact cut key and how many of its ties to keep
//   compact (tiles x rows) ascending positions, via a decoupled look-back
//
// Only the scan reads the 32 B/token index; the row kernel and the
// compaction read the row's 4 B/token logits once each.  Level-1 masses are taken relative
// to each bucket's upper bound - a data-independent reference, so tile
// histograms add without knowing the maximum - and rescaled to the top
// bucket's bound R when the row kernel reads them; later levels use R
// directly.  The row kernel zeroes the row's level-1 histogram after reading
// it, so a workspace that starts zero-filled stays reusable.
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
    if (j < a.n) VecLoad<T, 16, true>::run(a.k_idx, (krow + j) * 16, kv[i]);
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

// ------------------------------------------------------------------ row
constexpr int kRowThreads = 1024;

struct FindScratch {
  double scan_d[kRowThreads / 64];
  int64_t scan_i[kRowThreads / 64];
  int top, bm, bc;
  double bm_w, bc_w;          // mass above the crossing buckets
  int64_t bm_c, bc_c;         // count above the crossing buckets
};

// Cut of one radix level from the LDS histogram (s_c counts, s_w masses) of
// the keys under the current prefix: finds the bucket holding the cut under
// the live criteria, folds every bucket above it into the row state, and at
// level 3 fixes the cut key and the number of its ties to keep.
template <int LEVEL, bool MASS>
__device__ void find_cut(const SelectArgs& a, const uint32_t* s_c, double* s_w, RowState& st,
                         FindScratch& fs) {
  constexpr int NT = kRowThreads;
  constexpr int NB = (LEVEL == 3) ? 256 : 4096;
  constexpr int PER = (NB >= NT) ? NB / NT : 1;     // buckets per owning thread
  constexpr int BITS = (NB == 4096) ? 12 : 8;
  const int tid = threadIdx.x;
  const bool owns = PER * tid < NB;
  if (tid == 0) { fs.top = -1; fs.bm = -1; fs.bc = -1; }
  __syncthreads();
  if (LEVEL == 1 && MASS) {
    // reference R = upper bound of the highest non-empty bucket
    for (int i = tid; i < NB; i += NT) if (s_c[i]) atomicMax(&fs.top, i);
    __syncthreads();
    const double R = bucket_hi((uint32_t)max(fs.top, 0), 20);
    for (int i = tid; i < NB; i += NT)
      if (s_c[i]) s_w[i] = s_w[i] * exp(bucket_hi((uint32_t)i, 20) - R);
    if (tid == 0) st.R = R;
    __syncthreads();
  }
  // thread t owns buckets NB-1-PER*t ... NB-PER*t (descending key order)
  double tw = 0.0;
  int64_t tc = 0;
  if (owns) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int bk = NB - 1 - (PER * tid + k);
      if (MASS) tw += s_w[bk];
      tc += s_c[bk];
    }
  }
  double totw;
  int64_t totc;
  const double pre_w = block_exclusive_scan<double, NT>(tw, fs.scan_d, &totw);
  const int64_t pre_c = block_exclusive_scan<int64_t, NT>(tc, fs.scan_i, &totc);
  const int crit = st.crit;
  const double tmass = (LEVEL == 1) ? totw * a.top_p : st.target_mass;
  const double base_w = (LEVEL == 1) ? 0.0 : st.mass_above;
  const int64_t base_c = (LEVEL == 1) ? 0 : st.count_above;
  const int64_t tcount = st.target_count;
  if (owns) {
    double cw = base_w + pre_w;
    int64_t cc = base_c + pre_c;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int bk = NB - 1 - (PER * tid + k);
      const double nw = cw + (MASS ? s_w[bk] : 0.0);
      const int64_t nc = cc + s_c[bk];
      if ((crit & CRIT_MASS) && s_c[bk] && cw < tmass && nw >= tmass) {
        fs.bm = bk; fs.bm_w = cw; fs.bm_c = cc;
      }
      if ((crit & CRIT_COUNT) && s_c[bk] && cc < tcount && nc >= tcount) {
        fs.bc = bk; fs.bc_w = cw; fs.bc_c = cc;
      }
      cw = nw;
      cc = nc;
    }
  }
  __syncthreads();
  if (tid == 0) {
    if (LEVEL == 1) st.target_mass = tmass;
    const bool m_on = (crit & CRIT_MASS) != 0, c_on = (crit & CRIT_COUNT) != 0;
    int bm = fs.bm, bc = fs.bc;
    double bm_w = fs.bm_w;
    int64_t bm_c = fs.bm_c;
    if (m_on && bm < 0 && LEVEL > 1) {
      // The previous level placed the crossing inside this prefix; a
      // last-place disagreement between the two levels' mass sums lands it on
      // the first or last non-empty bucket (rare: a serial walk is fine).
      int hi_b = -1, lo_b = -1;
      for (int bk = NB - 1; bk >= 0; --bk)
        if (s_c[bk]) { if (hi_b < 0) hi_b = bk; lo_b = bk; }
      bm = (base_w >= tmass) ? hi_b : lo_b;
      bm_w = base_w;
      bm_c = base_c;
      for (int bk = NB - 1; bk > bm && bm >= 0; --bk) { if (MASS) bm_w += s_w[bk]; bm_c += s_c[bk]; }
    }
    // the mass crossing decides unless the count crossing lies further down
    // the order (a lower bucket); both stay live while they share a bucket
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
    } else {
      // everything above the chosen bucket, as accumulated by the scan
      const bool from_mass = (bstar == bm) && m_on;
      const double above_w = from_mass ? bm_w : fs.bc_w;
      const int64_t above_c = from_mass ? bm_c : fs.bc_c;
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
  }
  __syncthreads();
}

constexpr int kRowU = 8;                              // float4 per thread per chunk
constexpr int kRowChunk = kRowThreads * kRowU * 4;    // tokens per chunk (32 per thread)

// Histogram of the next radix digit of the row's logits whose keys carry the
// current prefix (level 2: bits 19..8, level 3: bits 7..0).  Each thread
// issues its chunk's eight 16-byte loads before using any of them.
template <int LEVEL, bool MASS>
__device__ void level_hist(const SelectArgs& a, const float* lg, const RowState& st, uint32_t* s_c,
                           double* s_w) {
  constexpr int NB = (LEVEL == 2) ? 4096 : 256;
  constexpr int SHIFT = (LEVEL == 2) ? 8 : 0;
  constexpr int PSHIFT = (LEVEL == 2) ? 20 : 8;
  const int tid = threadIdx.x;
  for (int i = tid; i < NB; i += kRowThreads) { s_c[i] = 0; if (MASS) s_w[i] = 0.0; }
  __syncthreads();
  const uint32_t prefix = st.prefix;
  const double R = st.R;
  for (int c0 = 0; c0 < a.n; c0 += kRowChunk) {
    float4 v[kRowU];
#pragma unroll
    for (int k = 0; k < kRowU; ++k) {
      const int j = c0 + 4 * (tid + k * kRowThreads);   // < row_stride: in bounds
      v[k] = *reinterpret_cast<const float4*>(lg + j);
    }
#pragma unroll
    for (int k = 0; k < kRowU; ++k) {
      const int j = c0 + 4 * (tid + k * kRowThreads);
      const float vv[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t key = order_key(vv[i]);
        if (j + i < a.n && (key >> PSHIFT) == prefix) {
          const uint32_t bk = (key >> SHIFT) & (NB - 1);
          atomicAdd(&s_c[bk], 1u);
          if (MASS) atomicAdd(&s_w[bk], exp((double)vv[i] - R));
        }
      }
    }
  }
  __syncthreads();
}

constexpr int kCand = 8192;        // logits of the level-1 cut bucket kept in LDS

// Collect the logits of the level-1 cut bucket into LDS (order is free).
// Returns their number; more than kCand means they did not fit.
__device__ int collect_candidates(const SelectArgs& a, const float* lg, uint32_t prefix, float* cand,
                                  int* s_cnt) {
  const int tid = threadIdx.x;
  if (tid == 0) *s_cnt = 0;
  __syncthreads();
  for (int c0 = 0; c0 < a.n; c0 += kRowChunk) {
    float4 v[kRowU];
#pragma unroll
    for (int k = 0; k < kRowU; ++k) v[k] = *reinterpret_cast<const float4*>(lg + c0 + 4 * (tid + k * kRowThreads));
#pragma unroll
    for (int k = 0; k < kRowU; ++k) {
      const int j = c0 + 4 * (tid + k * kRowThreads);
      const float vv[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if ((j + i < a.n) && ((order_key(vv[i]) >> 20) == prefix)) {
          const int slot = atomicAdd(s_cnt, 1);
          if (slot < kCand) cand[slot] = vv[i];
        }
      }
    }
  }
  __syncthreads();
  return *s_cnt;
}

// Histogram of the next digit over the candidates whose keys carry the
// current prefix (level 2: bits 19..8 under the 12-bit prefix, level 3:
// bits 7..0 under the 24-bit prefix).
template <int LEVEL, bool MASS>
__device__ void cand_hist(const float* cand, int nc, const RowState& st, uint32_t* s_c, double* s_w) {
  constexpr int NB = (LEVEL == 2) ? 4096 : 256;
  constexpr int SHIFT = (LEVEL == 2) ? 8 : 0;
  constexpr int PSHIFT = (LEVEL == 2) ? 20 : 8;
  const int tid = threadIdx.x;
  for (int i = tid; i < NB; i += kRowThreads) { s_c[i] = 0; if (MASS) s_w[i] = 0.0; }
  __syncthreads();
  const uint32_t prefix = st.prefix;
  const double R = st.R;
  for (int i = tid; i < nc; i += kRowThreads) {
    const float l = cand[i];
    const uint32_t key = order_key(l);
    if ((key >> PSHIFT) == prefix) {
      const uint32_t bk = (key >> SHIFT) & (NB - 1);
      atomicAdd(&s_c[bk], 1u);
      if (MASS) atomicAdd(&s_w[bk], exp((double)l - R));
    }
  }
  __syncthreads();
}

// One workgroup per row: every radix level after the scan's, leaving the
// row's cut (key, ties to keep, count) in the workspace for the compaction.
template <bool MASS>
__global__ __launch_bounds__(kRowThreads) void select_row_kernel(SelectArgs a) {
  __shared__ uint32_t s_c[4096];
  __shared__ double s_w[MASS ? 4096 : 1];
  __shared__ FindScratch fs;
  __shared__ RowState st;
  __shared__ float s_cand[kCand];
  __shared__ int s_ncand;
  const int row = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) {
    RowState init{};
    init.target_count = a.target_count;
    init.crit = (MASS ? CRIT_MASS : 0) | (a.target_count > 0 ? CRIT_COUNT : 0);
    st = init;
  }
  // level 1: the row's histogram as merged by the scan, zeroed after use
  uint32_t* gc = a.cnt1 + (int64_t)row * 4096;
  double* gw = a.mass1 + (int64_t)row * 4096;
  uint32_t cv[4];
  double wv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    cv[k] = gc[tid + k * kRowThreads];
    wv[k] = MASS ? gw[tid + k * kRowThreads] : 0.0;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    s_c[tid + k * kRowThreads] = cv[k];
    if (MASS) s_w[tid + k * kRowThreads] = wv[k];
    gc[tid + k * kRowThreads] = 0;
    if (MASS) gw[tid + k * kRowThreads] = 0.0;
  }
  __syncthreads();
  find_cut<1, MASS>(a, s_c, s_w, st, fs);
  const float* lg = a.logits + (int64_t)row * a.row_stride;
  // levels 2 and 3 over the cut bucket's logits, gathered into LDS once (a
  // streaming pass per level when they do not fit)
  int nc = 0;
  if (!st.all) nc = collect_candidates(a, lg, st.prefix, s_cand, &s_ncand);
  const bool fits = nc <= kCand;
  if (!st.all) {
    if (fits) cand_hist<2, MASS>(s_cand, nc, st, s_c, s_w); else level_hist<2, MASS>(a, lg, st, s_c, s_w);
    find_cut<2, MASS>(a, s_c, s_w, st, fs);
  }
  if (!st.all) {
    if (fits) cand_hist<3, MASS>(s_cand, nc, st, s_c, s_w); else level_hist<3, MASS>(a, lg, st, s_c, s_w);
    find_cut<3, MASS>(a, s_c, s_w, st, fs);
  }
  if (tid == 0) a.state[row] = st;
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

hipError_t launch_select_lowrank(const SelectArgs& a, int dtype, hipStream_t s) {
  const int rows = a.B * a.groups.n;
  if (rows == 0) return hipSuccess;
  if (!a.select_all) {
    dim3 grid(a.tiles, rows);
    if (dtype == 0) {
      if (a.use_mass) hipLaunchKernelGGL((select_scan_kernel<bf16_t, true>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((select_scan_kernel<bf16_t, false>), grid, dim3(kThreads), 0, s, a);
    } else {
      if (a.use_mass) hipLaunchKernelGGL((select_scan_kernel<float, true>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((select_scan_kernel<float, false>), grid, dim3(kThreads), 0, s, a);
    }
    if (a.use_mass) hipLaunchKernelGGL((select_row_kernel<true>), dim3(rows), dim3(kRowThreads), 0, s, a);
    else hipLaunchKernelGGL((select_row_kernel<false>), dim3(rows), dim3(kRowThreads), 0, s, a);
  }
  hipLaunchKernelGGL(select_compact_kernel, dim3(a.tiles, rows), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
