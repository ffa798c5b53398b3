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
//   scan (2K-token tiles x rows)  logits to the workspace (4 B/token) + level-1
//                        histogram of counts and fp64 masses, merged into the
//                        row's histogram with atomics
//   row  (rows)          one 1024-thread workgroup per row: the level-1 cut
//                        from the merged histogram held in registers, then
//                        the logits of the cut bucket gathered into LDS and
//                        levels 2 and 3 over them (LDS histograms): the exact
//                        cut key and how many of its ties to keep
//   compact (tiles x rows) ascending positions, via a decoupled look-back
//
// Only the scan reads the 32 B/token index; the row kernel and the
// compaction read the row's 4 B/token logits once each.  Level-1 masses are taken relative
// to each bucket's upper bound - a data-independent reference, so tile
// histograms add without knowing the maximum - and rescaled to the top
// bucket's bound R when the row kernel reads them (the scan also records the
// row's largest key); later levels use R directly.  The row kernel zeroes the
// row's level-1 histogram and largest key after reading them, and the scan
// clears the compaction's look-back words, so a workspace that starts
// zero-filled stays reusable.
#include "args.hpp"
#include "common.hpp"

namespace sa {

constexpr int kTile = 1024;        // tokens per compaction workgroup
constexpr int kScanTile = 2048;    // tokens per scan workgroup (two compaction tiles)
constexpr int kThreads = 256;
constexpr int kPer = kTile / kThreads;
constexpr int kScanPer = kScanTile / kThreads;
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
// Raw 32-byte index rows of one token, requested before any is used.
template <typename T> struct IdxRow;
template <> struct IdxRow<bf16_t> {
  vl_u32x4 w[2];
  __device__ void load(const void* base, int64_t row) {
    const vl_u32x4* p = reinterpret_cast<const vl_u32x4*>(reinterpret_cast<const uint16_t*>(base) + row * 16);
    w[0] = __builtin_nontemporal_load(p);
    w[1] = __builtin_nontemporal_load(p + 1);
  }
  __device__ float dot(const float (&q)[16]) const {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t x = w[e >> 2][e & 3];
      acc = fmaf(q[2 * e], bf16_lo(x), acc);
      acc = fmaf(q[2 * e + 1], bf16_hi(x), acc);
    }
    return acc;
  }
};
template <> struct IdxRow<float> {
  vl_f32x4 w[4];
  __device__ void load(const void* base, int64_t row) {
    const vl_f32x4* p = reinterpret_cast<const vl_f32x4*>(reinterpret_cast<const float*>(base) + row * 16);
#pragma unroll
    for (int c = 0; c < 4; ++c) w[c] = __builtin_nontemporal_load(p + c);
  }
  __device__ float dot(const float (&q)[16]) const {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc = fmaf(q[e], w[e >> 2][e & 3], acc);
    return acc;
  }
};

template <typename T, bool MASS>
__global__ __launch_bounds__(kThreads) void select_scan_kernel(SelectArgs a) {
  __shared__ uint32_t lc[4096];
  __shared__ double lw[MASS ? 4096 : 1];
  __shared__ uint32_t s_kmax[kThreads / 64];
  const int row = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
  int b, g;
  row_coords(a, row, b, g);
  // the tile's index rows first (tokens past the end re-read the last one),
  // so their latency overlaps everything up to the first use
  const int64_t krow = ((int64_t)b * a.Hkv + g) * a.n_cap;
  IdxRow<T> kr[kScanPer];
#pragma unroll
  for (int i = 0; i < kScanPer; ++i)
    kr[i].load(a.k_idx, krow + min(tile * kScanTile + i * kThreads + tid, a.n - 1));

  for (int i = tid; i < 4096; i += kThreads) { lc[i] = 0; if (MASS) lw[i] = 0.0; }
  // the compaction's look-back words of this call start empty
  if (tid < kScanTile / kTile && tile * (kScanTile / kTile) + tid < a.tiles)
    a.lookback[(int64_t)row * a.tiles + tile * (kScanTile / kTile) + tid] = 0;

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
  lds_barrier();

  float* lg = a.logits + (int64_t)row * a.row_stride;
  uint32_t kmax = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    const int j = tile * kScanTile + i * kThreads + tid;
    if (j < a.n) {
      float l = kr[i].dot(qb) * 0.25f;
      if (l == 0.f) l = 0.f;                       // fold -0 into +0
      lg[j] = l;
      const uint32_t key = order_key(l);
      kmax = max(kmax, key);
      const uint32_t bk = key >> 20;
      atomicAdd(&lc[bk], 1u);
      if (MASS) atomicAdd(&lw[bk], exp((double)l - bucket_hi(bk, 20)));
    }
  }
  // the row's largest key (its top bucket's bound is the row kernel's
  // reference for the masses): one atomic per workgroup
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m));
  if ((tid & 63) == 0) s_kmax[tid >> 6] = kmax;
  __syncthreads();
  if (tid == 0) {
    uint32_t km = s_kmax[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) km = max(km, s_kmax[w]);
    if (km) atomicMax(a.maxkey + row, km);
  }
  merge_hist<4096>(lc, lw, a.cnt1 + (int64_t)row * 4096, a.mass1 + (int64_t)row * 4096, MASS);
}

// ------------------------------------------------------------------ row
constexpr int kRowThreads = 1024;
constexpr int kRowWaves = kRowThreads / 64;
constexpr int kRowU = 8;                              // float4 per thread per chunk
constexpr int kRowChunk = kRowThreads * kRowU * 4;    // tokens per chunk (32 per thread)
constexpr int kCand = 8192;        // logits of the level-1 cut bucket kept in LDS

typedef uint32_t sel_u32x4 __attribute__((ext_vector_type(4)));
typedef double sel_f64x2 __attribute__((ext_vector_type(2)));
typedef float sel_f32x4 __attribute__((ext_vector_type(4)));

// Buckets of one level where the mass and the count targets are crossed, as
// published by the threads that own them (-1: not crossed in this level).
struct Cross {
  int bm, bc;
  double bm_w, bc_w;          // mass above the crossing bucket
  int64_t bm_c, bc_c;         // count above the crossing bucket
};

struct RowShared {
  double wave_w[3][kRowWaves];     // per level: inclusive wave totals
  int64_t wave_c[3][kRowWaves];
  uint32_t cand_w[2][kRowWaves];   // candidate counts, alternating per chunk
  Cross x[3];
};

// A 32- or 64-bit value of one lane (the lane index is wave-uniform), or of
// the first active lane: the result lives in scalar registers.
template <typename T>
__device__ __forceinline__ T lane_value(T v, int src) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), src);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}
template <typename T>
__device__ __forceinline__ T uniform(T v) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}

// One radix level.  Thread t owns the PER buckets NB-1-PER*t ... NB-PER*t
// (descending key order), their counts c[] and masses w[] in registers.  The
// prefix above each thread's buckets comes from wave scans and, across the
// workgroup's waves, one barrier and a 16-lane scan of the wave totals (with
// ONE_WAVE a single wave owns every bucket and no barrier is needed).  The
// owners of the crossing buckets publish them and every thread takes the same
// decision, in scalar registers, into its copy of the row state `st`.  The
// histogram hc / hw in LDS is read only by the rare fallback below and, at
// level 3, for the tie count.
template <int LEVEL, bool MASS, int PER, int NB, bool ONE_WAVE>
__device__ __forceinline__ void cut_level(const SelectArgs& a, const uint32_t (&c)[PER],
                                          const double (&w)[PER], bool owns, RowState& st,
                                          RowShared& sh, const uint32_t* hc, const double* hw) {
  constexpr int BITS = (NB == 4096) ? 12 : 8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int owner = ONE_WAVE ? lane : tid;
  double tw = 0.0;
  int64_t tc = 0;
  if (owns) {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (MASS) tw += w[k];
      tc += c[k];
    }
  }
  const double iw = wave_inclusive_scan(tw);
  const int64_t ic = wave_inclusive_scan(tc);
  double pre_w, totw;
  int64_t pre_c, totc;
  if constexpr (ONE_WAVE) {
    pre_w = iw - tw;
    pre_c = ic - tc;
    totw = lane_value(iw, 63);
    totc = lane_value(ic, 63);
  } else {
    if (lane == 63) {
      sh.wave_w[LEVEL - 1][wid] = iw;
      sh.wave_c[LEVEL - 1][wid] = ic;
    }
    lds_barrier();
    // every 16-lane row holds the wave totals; their inclusive prefix
    double pw = sh.wave_w[LEVEL - 1][lane & 15];
    int64_t pc = sh.wave_c[LEVEL - 1][lane & 15];
    pw += dpp_move<0x111, 0xF>(pw); pc += dpp_move<0x111, 0xF>(pc);
    pw += dpp_move<0x112, 0xF>(pw); pc += dpp_move<0x112, 0xF>(pc);
    pw += dpp_move<0x114, 0xF>(pw); pc += dpp_move<0x114, 0xF>(pc);
    pw += dpp_move<0x118, 0xF>(pw); pc += dpp_move<0x118, 0xF>(pc);
    totw = lane_value(pw, kRowWaves - 1);
    totc = lane_value(pc, kRowWaves - 1);
    const double bw = wid ? lane_value(pw, wid - 1) : 0.0;
    const int64_t bcn = wid ? lane_value(pc, wid - 1) : 0;
    pre_w = bw + iw - tw;
    pre_c = bcn + ic - tc;
  }
  const int crit = st.crit;
  const double tmass = (LEVEL == 1) ? totw * a.top_p : st.target_mass;
  const double base_w = (LEVEL == 1) ? 0.0 : st.mass_above;
  const int64_t base_c = (LEVEL == 1) ? 0 : st.count_above;
  const int64_t tcount = st.target_count;
  // this thread's crossings, if any
  int my_bm = -1, my_bc = -1;
  double my_bm_w = 0.0, my_bc_w = 0.0;
  int64_t my_bm_c = 0, my_bc_c = 0;
  if (owns) {
    double cw = base_w + pre_w;
    int64_t cc = base_c + pre_c;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int bk = NB - 1 - (PER * owner + k);
      const double nw = cw + (MASS ? w[k] : 0.0);
      const int64_t nc = cc + c[k];
      if ((crit & CRIT_MASS) && c[k] && cw < tmass && nw >= tmass) { my_bm = bk; my_bm_w = cw; my_bm_c = cc; }
      if ((crit & CRIT_COUNT) && c[k] && cc < tcount && nc >= tcount) { my_bc = bk; my_bc_w = cw; my_bc_c = cc; }
      cw = nw;
      cc = nc;
    }
  }
  int bm, bc;
  double bm_w, bc_w;
  int64_t bm_c, bc_c;
  if constexpr (ONE_WAVE) {
    const uint64_t fm = __ballot(my_bm >= 0), fc = __ballot(my_bc >= 0);
    const int lm = fm ? __ffsll((unsigned long long)fm) - 1 : 0;
    const int lc = fc ? __ffsll((unsigned long long)fc) - 1 : 0;
    bm = fm ? lane_value(my_bm, lm) : -1;
    bm_w = lane_value(my_bm_w, lm);
    bm_c = lane_value(my_bm_c, lm);
    bc = fc ? lane_value(my_bc, lc) : -1;
    bc_w = lane_value(my_bc_w, lc);
    bc_c = lane_value(my_bc_c, lc);
  } else {
    Cross& x = sh.x[LEVEL - 1];
    if (my_bm >= 0) { x.bm = my_bm; x.bm_w = my_bm_w; x.bm_c = my_bm_c; }
    if (my_bc >= 0) { x.bc = my_bc; x.bc_w = my_bc_w; x.bc_c = my_bc_c; }
    lds_barrier();
    bm = uniform(x.bm);
    bm_w = uniform(x.bm_w);
    bm_c = uniform(x.bm_c);
    bc = uniform(x.bc);
    bc_w = uniform(x.bc_w);
    bc_c = uniform(x.bc_c);
  }
  if (LEVEL == 1) st.target_mass = tmass;
  const bool m_on = (crit & CRIT_MASS) != 0, c_on = (crit & CRIT_COUNT) != 0;
  if (LEVEL > 1 && m_on && bm < 0) {
    // The previous level placed the crossing inside this prefix; a last-place
    // disagreement between the two levels' mass sums lands it on the first or
    // last non-empty bucket (rare: a serial walk is fine).
    int hi_b = -1, lo_b = -1;
    for (int bk = NB - 1; bk >= 0; --bk)
      if (hc[bk]) { if (hi_b < 0) hi_b = bk; lo_b = bk; }
    bm = (base_w >= tmass) ? hi_b : lo_b;
    bm_w = base_w;
    bm_c = base_c;
    for (int bk = NB - 1; bk > bm && bm >= 0; --bk) { if (MASS) bm_w += hw[bk]; bm_c += hc[bk]; }
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
  if (bstar < 0) {                   // the target lies past the last token
    st.all = 1;                      // every key lies above cut_key 0
    st.m = a.n;
    st.cut_key = 0;
    st.need = 0;
    return;
  }
  const bool from_mass = (bstar == bm) && m_on;
  const double above_w = from_mass ? bm_w : bc_w;
  const int64_t above_c = from_mass ? bm_c : bc_c;
  const uint32_t prefix = (LEVEL == 1) ? (uint32_t)bstar : ((st.prefix << BITS) | (uint32_t)bstar);
  st.mass_above = above_w;
  st.count_above = above_c;
  st.crit = ncrit;
  st.prefix = prefix;
  if (LEVEL == 3) {
    const int64_t ties = hc[bstar];
    int64_t need = 1;
    if (ncrit & CRIT_MASS) {
      const double e = exp((double)key_to_float(prefix) - st.R);
      const double cn = ceil((tmass - above_w) / e);
      need = (cn >= (double)ties) ? ties : (cn <= 1.0 ? 1 : (int64_t)cn);
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

// Histogram of the next radix digit of the row's logits whose keys carry the
// current prefix (level 2: bits 19..8, level 3: bits 7..0), streamed from the
// workspace: the fallback when the cut bucket holds more than kCand logits.
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
  const int last = (int)a.row_stride - 4;
  for (int c0 = 0; c0 < a.n; c0 += kRowChunk) {
    sel_f32x4 v[kRowU];
#pragma unroll
    for (int k = 0; k < kRowU; ++k)
      v[k] = *reinterpret_cast<const sel_f32x4*>(lg + min(c0 + 4 * (tid + k * kRowThreads), last));
#pragma unroll
    for (int k = 0; k < kRowU; ++k) {
      const int j = c0 + 4 * (tid + k * kRowThreads);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t key = order_key(v[k][i]);
        if (j + i < a.n && (key >> PSHIFT) == prefix) {
          const uint32_t bk = (key >> SHIFT) & (NB - 1);
          atomicAdd(&s_c[bk], 1u);
          if (MASS) atomicAdd(&s_w[bk], exp((double)v[k][i] - R));
        }
      }
    }
  }
  __syncthreads();
}

// One workgroup per row: every radix level after the scan's, leaving the
// row's cut (key, ties to keep, count) in the workspace for the compaction.
// Every thread holds the row state; the barriers order LDS only, so the first
// chunk of logits, requested at the start, stays in flight through level 1.
template <bool MASS>
__global__ __launch_bounds__(kRowThreads) void select_row_kernel(SelectArgs a) {
  __shared__ uint32_t s_c[4096];                 // level-2 histogram
  __shared__ double s_w[MASS ? 4096 : 1];
  __shared__ uint32_t s_c3[256];                 // level-3 histogram
  __shared__ double s_w3[MASS ? 256 : 1];
  __shared__ float s_cand[kCand];
  __shared__ RowShared sh;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

  // level 1: this thread's four buckets of the histogram merged by the scan
  // (returned to zero here), and the row's largest key
  uint32_t* gc = a.cnt1 + (int64_t)row * 4096;
  double* gw = a.mass1 + (int64_t)row * 4096;
  const int b0 = 4092 - 4 * tid;                 // buckets b0 .. b0 + 3
  const sel_u32x4 c4 = *reinterpret_cast<const sel_u32x4*>(gc + b0);
  sel_f64x2 w4[2] = {{0.0, 0.0}, {0.0, 0.0}};
  if (MASS) {
    w4[0] = *reinterpret_cast<const sel_f64x2*>(gw + b0);
    w4[1] = *reinterpret_cast<const sel_f64x2*>(gw + b0 + 2);
  }
  const uint32_t mk = a.maxkey[row];
  // first chunk of the row's logits (addresses clamped into the row)
  const float* lg = a.logits + (int64_t)row * a.row_stride;
  const int last = (int)a.row_stride - 4;
  sel_f32x4 v[kRowU];
#pragma unroll
  for (int k = 0; k < kRowU; ++k)
    v[k] = *reinterpret_cast<const sel_f32x4*>(lg + min(4 * (tid + k * kRowThreads), last));
  *reinterpret_cast<sel_u32x4*>(gc + b0) = sel_u32x4{0u, 0u, 0u, 0u};
  if (MASS) {
    *reinterpret_cast<sel_f64x2*>(gw + b0) = sel_f64x2{0.0, 0.0};
    *reinterpret_cast<sel_f64x2*>(gw + b0 + 2) = sel_f64x2{0.0, 0.0};
  }
  for (int i = tid; i < 4096; i += kRowThreads) { s_c[i] = 0; if (MASS) s_w[i] = 0.0; }
  if (tid < 256) { s_c3[tid] = 0; if (MASS) s_w3[tid] = 0.0; }
  if (tid < 3) { sh.x[tid].bm = -1; sh.x[tid].bc = -1; }

  RowState st{};
  st.target_count = a.target_count;
  st.crit = (MASS ? CRIT_MASS : 0) | (a.target_count > 0 ? CRIT_COUNT : 0);
  // masses arrive relative to each bucket's upper bound; rescale them to the
  // top bucket's bound R
  const double R = bucket_hi(mk >> 20, 20);
  if (MASS) st.R = R;
  uint32_t c1[4];
  double w1[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int e = 3 - k;                           // bucket 4095 - 4 tid - k
    c1[k] = c4[e];
    const double wr = w4[e >> 1][e & 1];
    w1[k] = (MASS && c1[k]) ? wr * exp(bucket_hi((uint32_t)(b0 + e), 20) - R) : 0.0;
  }
  cut_level<1, MASS, 4, 4096, false>(a, c1, w1, true, st, sh, nullptr, nullptr);
  if (tid == 0) a.maxkey[row] = 0;                // every thread has used it

  // the logits of the level-1 cut bucket, gathered into LDS (ascending
  // positions per chunk; a block prefix of per-thread counts gives the slots)
  int nc = 0;
  if (!st.all) {
    const uint32_t pf = st.prefix;
    uint32_t total = 0;
    int it = 0;
    for (int c0 = 0; c0 < a.n; c0 += kRowChunk, ++it) {
      if (c0 > 0) {
#pragma unroll
        for (int k = 0; k < kRowU; ++k)
          v[k] = *reinterpret_cast<const sel_f32x4*>(lg + min(c0 + 4 * (tid + k * kRowThreads), last));
      }
      // bit 4k+i: value i of load k lies in the cut bucket (keys compared
      // branch-free; positions past the row's end are masked off after)
      const uint32_t kb = pf << 20;
      uint32_t mask = 0;
#pragma unroll
      for (int k = 0; k < kRowU; ++k) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = __float_as_uint(v[k][i]);
          const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
          mask |= (uint32_t)((key - kb) < 0x100000u) << (4 * k + i);
        }
      }
      const int rem = a.n - c0;
      if (rem < kRowChunk) {
        uint32_t valid = 0;
#pragma unroll
        for (int k = 0; k < kRowU; ++k) {
          const int nv = min(max(rem - 4 * (tid + k * kRowThreads), 0), 4);
          valid |= ((1u << nv) - 1u) << (4 * k);
        }
        mask &= valid;
      }
      const uint32_t cnt = __popc(mask);
      const uint32_t incl = wave_inclusive_scan(cnt);
      if (lane == 63) sh.cand_w[it & 1][wid] = incl;
      lds_barrier();
      uint32_t base = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w) {
        const uint32_t sc = sh.cand_w[it & 1][w];
        if (w < wid) base += sc;
        tot += sc;
      }
      if (mask) {
        uint32_t slot = total + base + incl - cnt;
#pragma unroll
        for (int k = 0; k < kRowU; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((mask >> (4 * k + i)) & 1u) {
              if (slot < (uint32_t)kCand) s_cand[slot] = v[k][i];
              ++slot;
            }
      }
      total += tot;
    }
    lds_barrier();
    nc = (int)total;
  }
  const bool fits = nc <= kCand;

  // level 2: bits 19..8 under the 12-bit prefix
  if (!st.all) {
    if (fits) {
      for (int i = tid; i < nc; i += kRowThreads) {
        const float l = s_cand[i];
        const uint32_t key = order_key(l);
        if ((key >> 20) == st.prefix) {
          const uint32_t bk = (key >> 8) & 4095u;
          atomicAdd(&s_c[bk], 1u);
          if (MASS) atomicAdd(&s_w[bk], exp((double)l - st.R));
        }
      }
      lds_barrier();
    } else {
      level_hist<2, MASS>(a, lg, st, s_c, s_w);
    }
    const sel_u32x4 cc = *reinterpret_cast<const sel_u32x4*>(s_c + b0);
    sel_f64x2 ww[2] = {{0.0, 0.0}, {0.0, 0.0}};
    if (MASS) {
      ww[0] = *reinterpret_cast<const sel_f64x2*>(s_w + b0);
      ww[1] = *reinterpret_cast<const sel_f64x2*>(s_w + b0 + 2);
    }
    uint32_t c2[4];
    double w2[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 3 - k;
      c2[k] = cc[e];
      w2[k] = MASS ? ww[e >> 1][e & 1] : 0.0;
    }
    cut_level<2, MASS, 4, 4096, false>(a, c2, w2, true, st, sh, s_c, s_w);
  }

  // level 3: bits 7..0 under the 24-bit prefix; the histogram by every
  // wave, the cut by wave 0 alone (lane l owns buckets 255-4l ... 252-4l)
  if (!st.all) {
    if (fits) {
      for (int i = tid; i < nc; i += kRowThreads) {
        const float l = s_cand[i];
        const uint32_t key = order_key(l);
        if ((key >> 8) == st.prefix) {
          atomicAdd(&s_c3[key & 255u], 1u);
          if (MASS) atomicAdd(&s_w3[key & 255u], exp((double)l - st.R));
        }
      }
      lds_barrier();
    } else {
      level_hist<3, MASS>(a, lg, st, s_c3, s_w3);
    }
  }
  if (wid != 0) return;
  if (!st.all) {
    const int b3 = 252 - 4 * lane;
    const sel_u32x4 cc = *reinterpret_cast<const sel_u32x4*>(s_c3 + b3);
    sel_f64x2 ww[2] = {{0.0, 0.0}, {0.0, 0.0}};
    if (MASS) {
      ww[0] = *reinterpret_cast<const sel_f64x2*>(s_w3 + b3);
      ww[1] = *reinterpret_cast<const sel_f64x2*>(s_w3 + b3 + 2);
    }
    uint32_t c3[4];
    double w3[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int e = 3 - k;
      c3[k] = cc[e];
      w3[k] = MASS ? ww[e >> 1][e & 1] : 0.0;
    }
    cut_level<3, MASS, 4, 256, true>(a, c3, w3, true, st, sh, s_c3, s_w3);
  }
  if (lane == 0) a.state[row] = st;
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
  // their logits, requested first (in bounds: rows are whole tiles long)
  const float* lg = a.logits + (int64_t)row * a.row_stride;
  const vl_f32x4 lv = *reinterpret_cast<const vl_f32x4*>(lg + j0);
  if (a.select_all) {                          // every token: position j goes to slot j
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (j0 + i < a.n) a.sel_idx[orow + j0 + i] = j0 + i;
    if (tile == 0 && tid == 0) a.sel_count[(int64_t)b * a.Hkv + g] = a.n;
    return;
  }
  const RowState st = a.state[row];
  uint32_t strict_f = 0, tie_f = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int j = j0 + i;
    if (j >= a.n) continue;
    const uint32_t key = order_key(lv[i]);
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
    dim3 grid((a.n + kScanTile - 1) / kScanTile, rows);
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
