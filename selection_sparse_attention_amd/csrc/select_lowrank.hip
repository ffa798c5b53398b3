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
// histogram-based threshold): logits map to order-preserving 32-bit keys and
// the cut key is resolved digit by digit over histograms of counts and fp64
// masses.  One launch does the whole selection.  A row is split over W
// workgroups, each holding its tile of logits in registers from start to end
// (the logits never go to memory):
//
//   1. logits of the tile; LDS histogram of the top 12 key bits; merged into
//      the row's histogram in the workspace with returning atomics; arrival.
//   2. after every workgroup of the row has arrived, each reads the merged
//      histogram and takes the same level-1 decision: the bucket holding the
//      cut, with the count and mass above it.
//   3. the keys of that bucket's tokens (normally a few thousand per row) are
//      published to the row's candidate list; after a second arrival every
//      workgroup loads them into LDS and resolves the remaining 20 bits there
//      (two 10-bit digits): the exact cut key and how many of its ties to
//      keep.  A bucket with more than kCap tokens takes one more global round
//      (bits 19..8), then candidates or a last global round (bits 7..0).
//   4. compaction: each workgroup publishes its (above-cut, tie) counts in a
//      64-bit slot, sums its predecessors' slots and writes its selected
//      positions in ascending order.
//   5. the last workgroup of the row to leave writes sel_count (-1 when a
//      wait timed out) and returns the row's histograms, counters and slots to
//      zero, so a workspace that starts zero-filled stays reusable.
//
// Everything that crosses workgroups goes through agent-scope atomics
// (coherent across the dies' L2 caches): histogram adds and candidate writes
// return values that are consumed before the arrival is signalled, so they
// are performed by then, and every read of such data is an agent-coherent
// (sc1) load.  No fence is used.  A workgroup waits only for workgroups of
// its own row, and the host keeps W within what the device runs at once (see
// the launcher), so every wait ends; each is bounded anyway by a spin limit.
//
// Level-1 masses are accumulated relative to each bucket's upper bound (a
// data-independent reference, so tiles add without knowing the maximum) and
// rescaled to R = the upper bound of the row's highest non-empty bucket when
// the merged histogram is read; later digits use R directly.
#include "args.hpp"
#include "common.hpp"
#include "index_project.hpp"

namespace sa {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kNB1 = 4096;          // level-1 and level-2 buckets (12 bits)
constexpr int kNB3 = 256;           // level-3 buckets (8 bits)
constexpr int kNBL = 1024;          // local candidate digits (10 bits)
constexpr uint64_t kSlotFlag = 1ull << 63;

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

// Agent-coherent loads through a buffer resource (sc1: not served from a
// die's possibly stale cache lines).
constexpr int kSc1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ vl_u32x4 ld_sc1_u32x4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(vl_u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}

// Make the compiler wait for a value (a returned atomic) before going on.
__device__ __forceinline__ void consume(uint32_t v) { asm volatile("" ::"v"(v)); }

// ------------------------------------------------------------------ index rows
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

// ------------------------------------------------------------------ shared state
// The cut as it is resolved, held identically by every thread.
struct Cut {
  double R;             // reference logit: masses are exp(l - R)
  double tmass;         // p * total mass
  double above_w;       // mass of the tokens above the current prefix
  int64_t above_c;      // tokens above the current prefix
  int64_t tcount;       // count target (k, or min_tokens)
  uint32_t prefix;      // the key's top `bits` bits
  int bits;             // bits fixed so far
  int crit;             // live criteria
  int all;              // every token is selected
  uint32_t in_count;    // tokens carrying the prefix
  int32_t need;         // final: ties kept among keys == prefix (bits == 32)
};

// Crossing of one criterion inside a digit, as published by its owner.
struct Cross {
  int b;                // bucket, -1: none
  double w;             // mass above it
  int64_t c;            // count above it
};

template <bool MASS>
struct SelShared {
  union {
    struct {            // histogram of a global digit
      uint32_t c[kNB1];
      double m[MASS ? kNB1 : 1];
    } h;
    struct {            // the exchange: every workgroup's counts, the candidates, local digits
      uint32_t key[kCap];
      uint32_t c[kNBL];
      double m[MASS ? kNBL : 1];
      uint32_t strict[kMaxSelW];   // above-prefix tokens of each workgroup
      uint32_t base[kMaxSelW + 1]; // exclusive prefix of the candidate counts
    } r;
  } u;
  double wave_w[kWaves];
  int64_t wave_c[kWaves];
  Cross xm, xc;
  uint32_t top;
  uint32_t cnt_s[16][kWaves], cnt_t[16][kWaves];
  uint32_t red[2][kWaves];
  uint32_t small[64];   // the last few candidates, for the single-wave cut
  uint32_t n_small;
  Cut fin;              // the single-wave cut, for every thread
  int bad;              // a wait of this workgroup timed out
  int err_any;          // some workgroup of the row reported a timed-out wait
  int last;             // this workgroup left the row last
};

// Wave 0: wait until each of the row's W words reaches `atleast` (returns
// false when a poll runs past the spin limit; a negative limit fails at once).
__device__ bool wait_round(const uint32_t* slots, int W, uint32_t atleast, int limit) {
  const int lane = threadIdx.x & 63;
  bool ok = limit >= 0;
  for (int base = 0; base < W && ok; base += 64) {
    const int i = base + lane;
    if (i < W) {
      int spins = 0;
      while (ld_agent(slots + i) < atleast) {
        if (++spins > limit) { ok = false; break; }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    ok = __ballot(!ok) == 0;
  }
  return ok;
}

// Position-order ranks (token j0 + i * 256 + tid) of the flagged tokens of a
// workgroup, for two flag sets at once (one pair of barriers): ra[i] / rb[i]
// for this thread's token i, and the workgroup's totals ta / tb.
template <int PER>
__device__ __forceinline__ void wg_ranks2(uint32_t fa, uint32_t fb, uint32_t (&ra)[PER],
                                          uint32_t (&rb)[PER], uint32_t& ta, uint32_t& tb,
                                          uint32_t (*ca)[kWaves], uint32_t (*cb)[kWaves]) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t ba[PER], bb[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    ba[i] = __ballot((fa >> i) & 1u);
    bb[i] = __ballot((fb >> i) & 1u);
    if (lane == 0) { ca[i][wid] = (uint32_t)__popcll(ba[i]); cb[i][wid] = (uint32_t)__popcll(bb[i]); }
  }
  __syncthreads();
  uint32_t runa = 0, runb = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    uint32_t bfa = 0, bfb = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t x = ca[i][w], y = cb[i][w];
      if (w < wid) { bfa += x; bfb += y; }
    }
    ra[i] = runa + bfa + (uint32_t)__popcll(ba[i] & lt);
    rb[i] = runb + bfb + (uint32_t)__popcll(bb[i] & lt);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) { runa += ca[i][w]; runb += cb[i][w]; }
  }
  __syncthreads();
  ta = runa;
  tb = runb;
}

// Block-wide inclusive prefix (thread order) of one double and one int64 with
// their block totals; LDS-only barriers.
template <bool MASS>
__device__ __forceinline__ void block_scan2(double tw, int64_t tc, SelShared<MASS>& sh, double& pre_w,
                                            int64_t& pre_c, double& tot_w, int64_t& tot_c) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const double iw = MASS ? wave_inclusive_scan(tw) : 0.0;
  const int64_t ic = wave_inclusive_scan(tc);
  if (lane == 63) { sh.wave_w[wid] = iw; sh.wave_c[wid] = ic; }
  lds_barrier();
  double bw = 0.0, aw = 0.0;
  int64_t bc = 0, ac = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const double x = MASS ? sh.wave_w[w] : 0.0;
    const int64_t y = sh.wave_c[w];
    if (w < wid) { bw += x; bc += y; }
    aw += x;
    ac += y;
  }
  pre_w = bw + iw - tw;
  pre_c = bc + ic - tc;
  tot_w = aw;
  tot_c = ac;
}

// One digit of the cut.  Thread t owns the PER buckets NB-1-PER*t ...
// NB-PER*t (descending key order) with counts c[] and masses w[] (relative to
// R); hc / hm hold the same digit's histogram in LDS (bucket i at index i),
// read only by the rare fallback below.  `first` marks level 1, where the
// mass target is p times the total.  Every thread ends with the same cut.
// (The state goes in and out by value: written through a reference, two of
// its fields set on different paths got merged into one store through a
// pointer, which kept the whole state in scratch memory.)
template <int NB, bool MASS>
__device__ __forceinline__ Cut cut_digit(const SelectArgs& a, const uint32_t (&c)[NB / kThreads],
                                         const double (&w)[NB / kThreads], bool first, Cut ct,
                                         SelShared<MASS>& sh, int dbits, const uint32_t* hc,
                                         const double* hm) {
  constexpr int PER = NB / kThreads;
  const int tid = threadIdx.x;
  double tw = 0.0;
  int64_t tc = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) { if (MASS) tw += w[k]; tc += c[k]; }
  double pre_w, tot_w;
  int64_t pre_c, tot_c;
  block_scan2<MASS>(tw, tc, sh, pre_w, pre_c, tot_w, tot_c);
  if (first && MASS) ct.tmass = tot_w * a.top_p;
  const double tmass = ct.tmass;
  const int64_t tcount = ct.tcount;
  const int crit = ct.crit;
  if (tid == 0) { sh.xm.b = -1; sh.xc.b = -1; }
  lds_barrier();
  {
    double cw = ct.above_w + pre_w;
    int64_t cc = ct.above_c + pre_c;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int bk = NB - 1 - (PER * tid + k);
      const double nw = cw + (MASS ? w[k] : 0.0);
      const int64_t nc = cc + c[k];
      if ((crit & CRIT_MASS) && c[k] && cw < tmass && nw >= tmass) { sh.xm.b = bk; sh.xm.w = cw; sh.xm.c = cc; }
      if ((crit & CRIT_COUNT) && c[k] && cc < tcount && nc >= tcount) { sh.xc.b = bk; sh.xc.w = cw; sh.xc.c = cc; }
      cw = nw;
      cc = nc;
    }
  }
  lds_barrier();
  Cross xm = sh.xm, xc = sh.xc;
  const bool m_on = (crit & CRIT_MASS) != 0, c_on = (crit & CRIT_COUNT) != 0;
  if (!first && m_on && xm.b < 0) {
    // the previous digit placed the mass crossing inside this prefix; a
    // last-place disagreement between the two digits' sums puts it on the
    // first or last non-empty bucket here (rare: a serial walk is fine)
    const bool above = ct.above_w >= tmass;
    int hi_b = -1, lo_b = -1;
    for (int bk = NB - 1; bk >= 0; --bk)
      if (hc[bk]) { if (hi_b < 0) hi_b = bk; lo_b = bk; }
    xm.b = above ? hi_b : lo_b;
    xm.w = ct.above_w;
    xm.c = ct.above_c;
    for (int bk = NB - 1; bk > xm.b && xm.b >= 0; --bk) { if (MASS) xm.w += hm[bk]; xm.c += hc[bk]; }
  }
  // the mass crossing decides unless the count crossing lies further down
  // the order (a lower bucket); both stay live while they share a bucket
  int bstar, ncrit;
  if (m_on && c_on) {
    const bool mass_wins = (xc.b < 0) || (xm.b >= 0 && xm.b < xc.b);
    const bool count_wins = (xm.b >= 0) && (xc.b >= 0) && (xc.b < xm.b);
    bstar = count_wins ? xc.b : xm.b;
    ncrit = mass_wins ? CRIT_MASS : (count_wins ? CRIT_COUNT : (CRIT_MASS | CRIT_COUNT));
  } else {
    bstar = m_on ? xm.b : xc.b;
    ncrit = crit;
  }
  if (bstar < 0) {             // the target lies past the last token
    ct.all = 1;
    return ct;
  }
  const bool from_mass = (bstar == xm.b) && m_on;
  ct.above_w = from_mass ? xm.w : xc.w;
  ct.above_c = from_mass ? xm.c : xc.c;
  ct.crit = ncrit;
  ct.prefix = (ct.bits == 0) ? (uint32_t)bstar : ((ct.prefix << dbits) | (uint32_t)bstar);
  ct.bits += dbits;
  // the chosen bucket's count: its owner's c[] entry, through LDS
  const int owner = (NB - 1 - bstar) / PER, k = (NB - 1 - bstar) % PER;
  if (tid == owner) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) if (q == k) v = c[q];
    sh.top = v;
  }
  lds_barrier();
  ct.in_count = sh.top;
  lds_barrier();
  if (ct.bits == 32) {
    // every token left carries the same key: how many of them to keep
    const int64_t ties = ct.in_count;
    int64_t need = 1;
    if (ncrit & CRIT_MASS) {
      const double e = exp((double)key_to_float(ct.prefix) - ct.R);
      const double cn = ceil((tmass - ct.above_w) / e);
      need = (cn >= (double)ties) ? ties : (cn <= 1.0 ? 1 : (int64_t)cn);
    }
    if (ncrit & CRIT_COUNT) {
      const int64_t nc = tcount - ct.above_c;
      need = need > nc ? need : nc;
    }
    if (need > ties) need = ties;
    if (need < 1) need = 1;
    ct.need = (int32_t)need;
  }
  return ct;
}

// A double held by one lane (the lane index is wave-uniform).
__device__ __forceinline__ double lane_f64(double v, int src) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), src);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// The remaining digits of the cut when at most 64 of the C candidate keys in
// LDS carry the current prefix: wave 0 sorts them (descending, a bitonic
// network over the lanes) and walks them in order with the rules of
// cut_digit: the lower of the live crossings decides, and at its key the
// tie count follows from the mass of one tie or from the count target.
template <bool MASS>
__device__ Cut cut_small(const SelectArgs& a, Cut ct, SelShared<MASS>& sh, int C) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int pb = ct.bits;
  const uint32_t pf = ct.prefix;
  if (tid == 0) sh.n_small = 0;
  lds_barrier();
  for (int i = tid; i < C; i += kThreads) {
    const uint32_t k = sh.u.r.key[i];
    if ((k >> (32 - pb)) == pf) {
      const uint32_t slot = atomicAdd(&sh.n_small, 1u);
      if (slot < 64u) sh.small[slot] = k;
    }
  }
  lds_barrier();
  if (tid < 64) {
    const int n = (int)min(sh.n_small, 64u);
    uint32_t k = lane < n ? sh.small[lane] : 0u;          // 0: no key (below every real one)
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)k, stride);
        const bool desc = (lane & size) == 0 || size == 64;
        const bool low = (lane & stride) == 0;
        k = (low == desc) ? max(k, o) : min(k, o);
      }
    }
    const bool valid = lane < n;
    const double e = (MASS && valid) ? exp((double)key_to_float(k) - ct.R) : 0.0;
    const double incl_w = MASS ? wave_inclusive_scan(e) : 0.0;
    const double before_w = ct.above_w + incl_w - e;
    const int64_t before_c = ct.above_c + lane;
    const bool m_on = (ct.crit & CRIT_MASS) != 0, c_on = (ct.crit & CRIT_COUNT) != 0;
    const uint64_t mx = __ballot(MASS && m_on && valid && before_w < ct.tmass && before_w + e >= ct.tmass);
    const uint64_t cx = __ballot(c_on && valid && before_c < ct.tcount && before_c + 1 >= ct.tcount);
    int lm = -1, lc = -1;
    if (m_on) lm = mx ? __ffsll((unsigned long long)mx) - 1 : (ct.above_w >= ct.tmass ? 0 : n - 1);
    if (c_on) lc = cx ? __ffsll((unsigned long long)cx) - 1 : (n - 1);
    const int ls = max(lm, lc);
    const uint32_t ks = (uint32_t)__builtin_amdgcn_readlane((int)k, max(ls, 0));
    const bool mass_live = m_on && lm >= 0 && (uint32_t)__builtin_amdgcn_readlane((int)k, lm) == ks;
    const bool count_live = c_on && lc >= 0 && (uint32_t)__builtin_amdgcn_readlane((int)k, lc) == ks;
    const uint64_t tie = __ballot(valid && k == ks);
    const int f = tie ? __ffsll((unsigned long long)tie) - 1 : 0;
    const int64_t ties = __popcll(tie);
    Cut r = ct;
    r.above_c = ct.above_c + f;
    r.above_w = MASS ? lane_f64(before_w, f) : 0.0;
    r.prefix = ks;
    r.bits = 32;
    r.in_count = (uint32_t)ties;
    r.crit = (mass_live ? CRIT_MASS : 0) | (count_live ? CRIT_COUNT : 0);
    int64_t need = 1;
    if (mass_live) {
      const double et = exp((double)key_to_float(ks) - ct.R);
      const double cn = ceil((ct.tmass - r.above_w) / et);
      need = (cn >= (double)ties) ? ties : (cn <= 1.0 ? 1 : (int64_t)cn);
    }
    if (count_live) {
      const int64_t nc = ct.tcount - r.above_c;
      need = need > nc ? need : nc;
    }
    if (need > ties) need = ties;
    if (need < 1) need = 1;
    r.need = (int32_t)need;
    if (ls < 0) r.all = 1;                               // no live criterion (cannot happen)
    if (lane == 0) sh.fin = r;
  }
  lds_barrier();
  return sh.fin;
}

// The fused append of one row (bf16 caches): the row's G <= 16 query heads
// projected into qrows (every workgroup; the first also stores q_idx) and,
// in the workgroup holding token n - 1, that token's index key into knew
// (bf16 bits) and k_idx - the index build's projection step by step, so the
// same bits.  Wave 0 issues every load (query rows, the key row, both
// projectors) before the first product; the other waves return at once and
// wait at the caller's barrier.
template <int D>
__device__ __forceinline__ void fused_append(const SelectArgs& a, int b, int g, int wg, float* qrows,
                                             uint16_t* knew) {
  if ((threadIdx.x >> 6) != 0) return;
  const int lane = threadIdx.x & 63, col = lane & 15, kb = lane >> 4;
  const int kvg = g / a.kv_div;                              // KV group within the sequence
  const int64_t qrow0 = (int64_t)b * a.Hq + (int64_t)g * a.G;
  const int64_t krow0 = ((int64_t)b * (a.Hkv / a.kv_div) + kvg) * a.n_cap;
  const bool key = wg == a.W - 1;
  vl_u32x4 qa[D / 32], ka[D / 32];
  ProjSlices<D> pq, pk;
  load_row_slices<D>(a.q_pre, qrow0, 0, a.G, qa);
  pq.load(a.proj_q + (int64_t)kvg * 16 * D);
  if (key) {
    load_row_slices<D>(a.k_pre, krow0, a.n - 1, a.n, ka);
    pk.load(a.proj_k + (int64_t)kvg * 16 * D);
  }
  {
    ProjParts<D> pp;
    pp.split(pq);
    const ix_f32x4 c = pp.tile(qa);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * kb + i;
      if (r < a.G) {
        qrows[r * 16 + col] = c[i];
        if (wg == 0) a.q_idx_w[(qrow0 + r) * 16 + col] = c[i];
      }
    }
  }
  if (key) {
    ProjParts<D> pp;
    pp.split(pk);
    const ix_f32x4 c = pp.tile(ka);
    if (kb == 0) {                                          // row n - 1: lanes 0-15, first value
      const uint16_t h = f32_to_bf16(c[0]);
      knew[col] = h;
      reinterpret_cast<uint16_t*>(a.k_idx_w)[(krow0 + a.n - 1) * 16 + col] = h;
    }
  }
}

// ------------------------------------------------------------------ the kernel
template <typename T, bool MASS, int PER>
__global__ __launch_bounds__(kThreads) void select_fused_kernel(SelectArgs a) {
  __shared__ SelShared<MASS> sh;
  __shared__ float s_qrows[16 * 16];       // fused append: the row's query heads' q_idx
  __shared__ uint16_t s_knew[16];          // fused append: token n - 1's index key
  const int row = blockIdx.y, wg = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  int b, g;
  row_coords(a, row, b, g);
  const int W = a.W;
  constexpr int TILE = kThreads * PER;
  const int j0 = wg * TILE;
  const int64_t orow = ((int64_t)b * a.Hkv + g) * a.n_cap;
  uint32_t* ctl = a.ctl + (int64_t)row * kCtlWords;
  uint32_t* slot_a = a.slot_a + (int64_t)row * kMaxSelW;
  uint64_t* slot_b = a.slot_b + (int64_t)row * kMaxSelW;
  uint32_t* cand_row = a.cand + (int64_t)row * a.cand_stride;
  uint32_t sink = 0;          // returned atomic values, consumed before a flag is raised

  // ---- 1. logits in registers, as order keys (token j0 + i * 256 + tid; a
  // key maps back to its logit exactly)
  uint32_t key[PER];
  {
    float qb[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) qb[c] = 0.f;
    const int64_t krow = (((int64_t)b * a.Hkv + g) / a.kv_div) * a.n_cap;
    constexpr int BATCH = PER < 8 ? PER : 8;
#pragma unroll
    for (int i0 = 0; i0 < PER; i0 += BATCH) {
      IdxRow<T> kr[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i)
        kr[i].load(a.k_idx, krow + min(j0 + (i0 + i) * kThreads + tid, a.n - 1));
      if (i0 == 0) {
        bool fused = false;
        // (4096-token tiles with masses would spill with it: the host
        // appends separately there)
        if constexpr (sizeof(T) == 2 && (PER <= 8 || !MASS)) {
          if (a.append) {
            // the projections overlap the index rows already in flight
            if (a.d == 128) fused_append<128>(a, b, g, wg, s_qrows, s_knew);
            else fused_append<64>(a, b, g, wg, s_qrows, s_knew);
            __syncthreads();
            for (int hh = 0; hh < a.G; ++hh) {
#pragma unroll
              for (int c = 0; c < 16; ++c) qb[c] += s_qrows[hh * 16 + c];
            }
            fused = true;
          }
        }
        if (!fused) {
          for (int hh = 0; hh < a.G; ++hh) {
            const float* qp = a.q_idx + ((int64_t)b * a.Hq + g * a.G + hh) * 16;
#pragma unroll
            for (int c = 0; c < 16; ++c) qb[c] += qp[c];
          }
        }
        const float invG = 1.0f / (float)a.G;
#pragma unroll
        for (int c = 0; c < 16; ++c) qb[c] *= invG;
      }
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        if constexpr (sizeof(T) == 2 && (PER <= 8 || !MASS)) {
          // token n - 1 under the fused append: its key from the projection
          // (the row loaded from k_idx predates it)
          if (a.append && j0 + (i0 + i) * kThreads + tid == a.n - 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              kr[i].w[e >> 2][e & 3] = (uint32_t)s_knew[2 * e] | ((uint32_t)s_knew[2 * e + 1] << 16);
          }
        }
        float l = kr[i].dot(qb) * 0.25f;
        if (l == 0.f) l = 0.f;                  // fold -0 into +0
        const bool valid = j0 + (i0 + i) * kThreads + tid < a.n;
        key[i0 + i] = valid ? order_key(l) : 0u;   // key 0: no token (below every real key)
      }
    }
  }
  auto valid = [&](int i) __attribute__((always_inline)) { return j0 + i * kThreads + tid < a.n; };

  Cut ct{};
  ct.tcount = a.target_count;
  ct.crit = (MASS ? CRIT_MASS : 0) | (a.target_count > 0 ? CRIT_COUNT : 0);
  ct.all = a.select_all;
  int rounds = 0;             // global digits taken (1..3)
  if (tid == 0) { sh.bad = 0; sh.err_any = 0; sh.last = 0; }
  __syncthreads();

  // ---- 2. one global digit: histogram of the tokens under the current
  // prefix, merged, flagged, waited for, read back and cut
  auto global_round = [&](int level) __attribute__((always_inline)) {
    const int NB = (level == 3) ? kNB3 : kNB1;
    const int shift = (level == 1) ? 20 : (level == 2 ? 8 : 0);
    const int pbits = ct.bits;
    const uint32_t prefix = ct.prefix;
    for (int i = tid; i < NB; i += kThreads) { sh.u.h.c[i] = 0; if (MASS) sh.u.h.m[i] = 0.0; }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t k = key[i];
      const bool in = valid(i) && (pbits == 0 || (k >> (32 - pbits)) == prefix);
      if (in) {
        const uint32_t bk = (k >> shift) & (uint32_t)(NB - 1);
        atomicAdd(&sh.u.h.c[bk], 1u);
        if (MASS) {
          const double ref = (level == 1) ? bucket_hi(bk, 20) : ct.R;
          atomicAdd(&sh.u.h.m[bk], exp((double)key_to_float(k) - ref));
        }
      }
    }
    lds_barrier();
    uint32_t* gc = a.hist_c + ((int64_t)row * 3 + (level - 1)) * kNB1;
    double* gm = a.hist_m + ((int64_t)row * 3 + (level - 1)) * kNB1;
    for (int i = tid; i < NB; i += kThreads) {
      const uint32_t cv = sh.u.h.c[i];
      if (cv) {
        sink ^= atomicAdd(gc + i, cv);
        if (MASS) sink ^= (uint32_t)__double_as_longlong(atomicAdd(gm + i, sh.u.h.m[i]));
      }
    }
    consume(sink);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(slot_a + wg, (uint32_t)level, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < 64) {
      const bool ok = wait_round(slot_a, W, (uint32_t)level, a.spin_limit);
      if (!ok && lane == 0) sh.bad = 1;
    }
    __syncthreads();
    // the merged histogram: thread t reads buckets NB-1-PER*t ... NB-PER*t,
    // the masses of its non-empty buckets only
    if (NB == kNB1) {
      constexpr int P1 = kNB1 / kThreads;     // 16
      uint32_t c[P1];
      double w[P1];
      const int lo = kNB1 - P1 * (tid + 1);   // lowest bucket of this thread
      const __amdgpu_buffer_rsrc_t rc = rsrc_of(gc);
      vl_u32x4 cv[P1 / 4];
#pragma unroll
      for (int q = 0; q < P1 / 4; ++q) cv[q] = ld_sc1_u32x4(rc, (lo + 4 * q) * 4);
#pragma unroll
      for (int k = 0; k < P1; ++k) {
        const int e = P1 - 1 - k;             // bucket lo + e, descending in k
        c[k] = cv[e >> 2][e & 3];
      }
#pragma unroll
      for (int k = 0; k < P1; ++k) w[k] = (MASS && c[k]) ? ld_agent(gm + lo + P1 - 1 - k) : 0.0;
      if (level == 1) {
        // R: the upper bound of the highest non-empty bucket
        int top = -1;
#pragma unroll
        for (int k = P1 - 1; k >= 0; --k) if (c[k]) top = kNB1 - 1 - (P1 * tid + k);
        if (tid == 0) sh.top = 0;
        lds_barrier();
        if (top >= 0) atomicMax(&sh.top, (uint32_t)top + 1u);
        lds_barrier();
        const uint32_t tb = sh.top;
        ct.R = tb ? bucket_hi(tb - 1, 20) : 0.0;
        if (MASS) {
          // rescale factors exp(hi(b) - R) of the non-empty buckets: listed in
          // LDS and computed a few per thread (the non-empty buckets bunch up
          // in a few threads' ranges), then read back by their owners
          uint32_t ne = 0;
#pragma unroll
          for (int k = 0; k < P1; ++k) ne |= (c[k] ? 1u : 0u) << k;
          uint32_t total;
          const uint32_t first_i = block_exclusive_scan<uint32_t, kThreads>(
              (uint32_t)__popc(ne), &sh.cnt_s[0][0], &total);
          uint32_t* list = sh.u.h.c;            // free: the tile's level-1 counts are merged
          double* fac = sh.u.h.m;
          {
            uint32_t i = first_i;
#pragma unroll
            for (int k = 0; k < P1; ++k)
              if ((ne >> k) & 1u) list[i++] = (uint32_t)(kNB1 - 1 - (P1 * tid + k));
          }
          lds_barrier();
          for (uint32_t i = tid; i < total; i += kThreads) fac[i] = exp(bucket_hi(list[i], 20) - ct.R);
          lds_barrier();
          {
            uint32_t i = first_i;
#pragma unroll
            for (int k = 0; k < P1; ++k)
              if ((ne >> k) & 1u) w[k] *= fac[i++];
          }
          lds_barrier();
        }
      } else {
        // the merged histogram in LDS, for the rare fallback walk
        lds_barrier();
#pragma unroll
        for (int k = 0; k < P1; ++k) {
          const int bk = kNB1 - 1 - (P1 * tid + k);
          sh.u.h.c[bk] = c[k];
          if (MASS) sh.u.h.m[bk] = w[k];
        }
        lds_barrier();
      }
      ct = cut_digit<kNB1, MASS>(a, c, w, level == 1, ct, sh, 12, sh.u.h.c, sh.u.h.m);
    } else {
      uint32_t c[1];
      double w[1];
      const int bk = kNB3 - 1 - tid;
      c[0] = ld_agent(gc + bk);
      w[0] = (MASS && c[0]) ? ld_agent(gm + bk) : 0.0;
      lds_barrier();
      sh.u.h.c[bk] = c[0];
      if (MASS) sh.u.h.m[bk] = w[0];
      lds_barrier();
      ct = cut_digit<kNB3, MASS>(a, c, w, false, ct, sh, 8, sh.u.h.c, sh.u.h.m);
    }
    rounds = level;
  };

  if (!ct.all) {
    global_round(1);
    while (!ct.all && ct.in_count > (uint32_t)kCap && ct.bits < 32) global_round(ct.bits == 12 ? 2 : 3);
  }

  // ---- 3. the exchange: every workgroup publishes how many of its tokens lie
  // above the prefix and, in position order, the keys of those that carry it
  // (none when all 32 bits are fixed: they are ties); after it, every
  // workgroup resolves the cut and knows what precedes its tiles
  uint32_t s_before = 0, a_before = 0, t_before = 0;
  if (rounds > 0) {
    const int pb = ct.bits;
    const uint32_t pf = ct.prefix;
    const bool keys = !ct.all && pb < 32;
    uint32_t fa = 0, fc = 0;                  // bit i: token i above / carrying the prefix
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (!valid(i)) continue;
      if (ct.all) { fa |= 1u << i; continue; }
      const uint32_t kp = key[i] >> (32 - pb);
      if (kp > pf) fa |= 1u << i;
      else if (kp == pf) fc |= 1u << i;
    }
    uint32_t ra[PER], rk[PER], n_above, n_cand;
    wg_ranks2<PER>(fa, fc, ra, rk, n_above, n_cand, sh.cnt_s, sh.cnt_t);
    if (keys) {
      uint32_t* region = cand_row + (int64_t)wg * TILE;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if ((fc >> i) & 1u)
          sink ^= __hip_atomic_exchange(region + rk[i], key[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    consume(sink);
    __syncthreads();
    if (tid == 0)
      __hip_atomic_store(slot_b + wg, kSlotFlag | ((uint64_t)sh.bad << 62) | ((uint64_t)n_above << 31) | n_cand,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every workgroup's counts, into LDS (wave 0)
    if (tid < 64) {
      bool ok = a.spin_limit >= 0;
      int err = 0;
      for (int base = 0; base < W; base += 64) {
        const int i = base + lane;
        uint64_t v = kSlotFlag;
        if (i < W && ok) {
          int spins = 0;
          v = ld_agent(slot_b + i);
          while (!(v & kSlotFlag)) {
            if (++spins > a.spin_limit) { ok = false; break; }
            __builtin_amdgcn_s_sleep(1);
            v = ld_agent(slot_b + i);
          }
        }
        if (i < W) {
          sh.u.r.strict[i] = ok ? (uint32_t)((v >> 31) & 0x7FFFFFFFu) : 0u;
          sh.u.r.base[i] = ok ? (uint32_t)(v & 0x7FFFFFFFu) : 0u;
          err |= (int)((v >> 62) & 1u);
        }
        ok = __ballot(!ok) == 0;
      }
      const bool any_err = __ballot(err != 0) != 0;
      if (lane == 0) {
        if (!ok) sh.bad = 1;
        if (any_err || !ok) sh.err_any = 1;
      }
    }
    __syncthreads();
    // exclusive prefixes of the candidate counts (wave 0, 64 at a time) and
    // the above-prefix tokens before this workgroup
    if (tid < 64) {
      uint32_t carry = 0, sb = 0;
      for (int base = 0; base < W; base += 64) {
        const int i = base + lane;
        const uint32_t cnt = i < W ? sh.u.r.base[i] : 0u;
        const uint32_t st = (i < wg) ? sh.u.r.strict[i] : 0u;
        const uint32_t inc = wave_inclusive_scan(cnt);
        if (i < W) sh.u.r.base[i] = carry + inc - cnt;
        carry += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
        uint32_t s2 = st;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) s2 += __shfl_xor(s2, o);
        sb += s2;
      }
      if (lane == 0) { sh.u.r.base[W] = carry; sh.red[0][0] = sb; }
    }
    __syncthreads();
    s_before = sh.red[0][0];
    const uint32_t C_all = sh.u.r.base[W];
    if (!ct.all && C_all != ct.in_count && tid == 0) sh.err_any = 1;   // the lists disagree
    if (keys) {
      // every candidate, region by region: position order
      // (wave w loads regions w, w + 4, ..., 64 keys per load, every load
      // issued before the first is used)
      const int C = (int)min(C_all, (uint32_t)kCap);
      {
        constexpr int kBatch = 8;
        for (int r0 = wid; r0 < W; r0 += kWaves * kBatch) {
          uint32_t v[kBatch];
          int dst[kBatch];
#pragma unroll
          for (int q = 0; q < kBatch; ++q) {
            const int r = r0 + q * kWaves;
            dst[q] = -1;
            v[q] = 0u;
            if (r < W) {
              const int lo = (int)sh.u.r.base[r], cnt = (int)sh.u.r.base[r + 1] - lo;
              for (int e = lane; e < cnt && lo + e < C; e += 64) {
                if (e >= 64) {                  // more than 64 keys in the region: rare
                  sh.u.r.key[lo + e] = ld_agent(cand_row + (int64_t)r * TILE + e);
                  continue;
                }
                v[q] = ld_agent(cand_row + (int64_t)r * TILE + e);
                dst[q] = lo + e;
              }
            }
          }
#pragma unroll
          for (int q = 0; q < kBatch; ++q)
            if (dst[q] >= 0) sh.u.r.key[dst[q]] = v[q];
        }
      }
      __syncthreads();
      // the remaining bits: 10 + 10 after 12, or 8 after 24, by LDS
      // histograms until at most 64 candidates are left, then by one wave
      while (ct.bits < 32 && !ct.all) {
        if (ct.in_count <= 64u) {
          ct = cut_small<MASS>(a, ct, sh, C);
          break;
        }
        const int rem = 32 - ct.bits;
        const int dbits = rem > 10 ? 10 : rem;
        const int shift = rem - dbits;
        const int NBd = 1 << dbits;
        const int pbd = ct.bits;
        const uint32_t pfd = ct.prefix;
        for (int i = tid; i < kNBL; i += kThreads) { sh.u.r.c[i] = 0; if (MASS) sh.u.r.m[i] = 0.0; }
        lds_barrier();
        for (int i = tid; i < C; i += kThreads) {
          const uint32_t k = sh.u.r.key[i];
          if ((k >> (32 - pbd)) == pfd) {
            const uint32_t bk = (k >> shift) & (uint32_t)(NBd - 1);
            atomicAdd(&sh.u.r.c[bk], 1u);
            if (MASS) atomicAdd(&sh.u.r.m[bk], exp((double)key_to_float(k) - ct.R));
          }
        }
        lds_barrier();
        if (NBd == kNBL) {
          constexpr int P = kNBL / kThreads;
          uint32_t c[P];
          double w[P];
#pragma unroll
          for (int k = 0; k < P; ++k) {
            const int bk = kNBL - 1 - (P * tid + k);
            c[k] = sh.u.r.c[bk];
            w[k] = MASS ? sh.u.r.m[bk] : 0.0;
          }
          ct = cut_digit<kNBL, MASS>(a, c, w, false, ct, sh, 10, sh.u.r.c, sh.u.r.m);
        } else {
          // 2^dbits buckets (dbits <= 8) fill the top of a 256-bucket digit
          uint32_t c[1];
          double w[1];
          const int bk = kNB3 - 1 - tid;
          c[0] = bk < NBd ? sh.u.r.c[bk] : 0u;
          w[0] = (MASS && bk < NBd) ? sh.u.r.m[bk] : 0.0;
          ct = cut_digit<kNB3, MASS>(a, c, w, false, ct, sh, dbits, sh.u.r.c, sh.u.r.m);
        }
      }
      // candidates of earlier workgroups above the cut, and ties among them
      const uint32_t cut = ct.prefix;
      const int mine = (int)min(sh.u.r.base[wg], (uint32_t)C);
      uint32_t na = 0, nt = 0;
      for (int i = tid; i < mine; i += kThreads) {
        const uint32_t k = sh.u.r.key[i];
        na += k > cut;
        nt += k == cut;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) { na += __shfl_xor(na, o); nt += __shfl_xor(nt, o); }
      if (lane == 0) { sh.red[0][wid] = na; sh.red[1][wid] = nt; }
      __syncthreads();
#pragma unroll
      for (int w = 0; w < kWaves; ++w) { a_before += sh.red[0][w]; t_before += sh.red[1][w]; }
    } else if (!ct.all) {
      t_before = sh.u.r.base[wg];              // every candidate is a tie
    }
  }

  // ---- 4. compaction: this workgroup's selected positions, ascending
  const uint32_t cut = ct.prefix;
  const int64_t need = ct.all ? 0 : ct.need;
  const int64_t m = ct.all ? (int64_t)a.n : ct.above_c + need;
  int bad = 0;
  {
    uint32_t fs = 0, ft = 0;                  // bit i: token i above the cut / a tie
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (!valid(i)) continue;
      if (ct.all || key[i] > cut) fs |= 1u << i;
      else if (key[i] == cut) ft |= 1u << i;
    }
    uint32_t rs[PER], rt[PER], ns, nt;
    wg_ranks2<PER>(fs, ft, rs, rt, ns, nt, sh.cnt_s, sh.cnt_t);   // (its barriers also publish sh.bad / sh.err_any)
    bad = sh.bad | sh.err_any;
    if (!bad) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int j = j0 + i * kThreads + tid;
        const int64_t sb = (int64_t)s_before + a_before + rs[i];
        const int64_t tb = (int64_t)t_before + rt[i];
        int64_t o = -1;
        if (ct.all) o = j;
        else if ((fs >> i) & 1u) o = sb + (tb < need ? tb : need);
        else if (((ft >> i) & 1u) && tb < need) o = sb + tb;
        if (o >= 0 && o < m && o < a.n_cap) a.sel_idx[orow + o] = j;
      }
    }
  }

  // ---- 5. this workgroup's share of the histograms back to zero (every
  // workgroup has read them: all have published in the exchange), then leave;
  // the last workgroup of the row out writes sel_count and clears the flags
  if (rounds > 0) {
    const int levels = bad ? 3 : rounds;
    for (int lvl = 0; lvl < levels; ++lvl) {
      const int NB = (lvl == 2) ? kNB3 : kNB1;
      uint32_t* gc = a.hist_c + ((int64_t)row * 3 + lvl) * kNB1;
      double* gm = a.hist_m + ((int64_t)row * 3 + lvl) * kNB1;
      for (int i = wg + tid * W; i < NB; i += kThreads * W) {
        gc[i] = 0u;
        if (MASS) gm[i] = 0.0;
      }
    }
  }
  if (tid == 0) {
    if (bad) sink ^= atomicOr(ctl + kCtlErr, 1u);
    consume(sink);
    const uint32_t old = atomicAdd(ctl + kCtlDepart, 1u);
    sh.last = (old == (uint32_t)W - 1);
  }
  __syncthreads();
  if (!sh.last) return;
  if (tid == 0) {
    const uint32_t err = ld_agent(ctl + kCtlErr);
    a.sel_count[(int64_t)b * a.Hkv + g] = err ? -1 : (int32_t)m;
  }
  __syncthreads();
  for (int i = tid; i < W; i += kThreads) { slot_a[i] = 0u; slot_b[i] = 0ull; }
  if (tid < kCtlWords) ctl[tid] = 0u;
}

hipError_t launch_select_lowrank(const SelectArgs& a, int dtype, int per, hipStream_t s) {
  const int rows = a.B * a.groups.n;
  if (rows == 0) return hipSuccess;
  dim3 grid(a.W, rows), block(kThreads);
#define SA_SEL(T_, M_, P_) hipLaunchKernelGGL((select_fused_kernel<T_, M_, P_>), grid, block, 0, s, a)
#define SA_SEL_P(T_, M_)                      \
  switch (per) {                              \
    case 8: SA_SEL(T_, M_, 8); break;         \
    case 16: SA_SEL(T_, M_, 16); break;       \
    default: return hipErrorInvalidValue;     \
  }
  if (dtype == 0) {
    if (a.use_mass) { SA_SEL_P(bf16_t, true) } else { SA_SEL_P(bf16_t, false) }
  } else {
    if (a.use_mass) { SA_SEL_P(float, true) } else { SA_SEL_P(float, false) }
  }
#undef SA_SEL_P
#undef SA_SEL
  return hipGetLastError();
}

// ------------------------------------------------------------------ visit order
// Rewrites each row's selected positions (sel_count[row] of them, at most
// kS2oMax) in visit order for the early-stop decode: index logit descending,
// then position ascending - the ranking the cut used, with every logit
// recomputed by the same arithmetic (so equal keys stay equal).  One
// workgroup per row: a stable least-significant-digit radix sort of the
// complemented order keys in LDS, four passes of 8 bits.  The list comes in
// ascending positions and every pass keeps the order of equal digits, so
// equal keys end in ascending positions.  In a pass, wave w takes elements
// [512 w, 512 w + 512) in rounds of 64: an element's rank among the wave's
// earlier elements with its digit comes from eight ballots and a running
// per-(wave, digit) count; the digit's offset adds every wave's count of
// smaller digits and the earlier waves' count of its own.
constexpr int kOrderThreads = 1024;
constexpr int kOrderWaves = kOrderThreads / 64;
constexpr int kOrderRounds = kS2oMax / kOrderThreads;   // rounds of 64 per wave

template <typename T>
__global__ __launch_bounds__(kOrderThreads) void select_order_kernel(SelectArgs a) {
  __shared__ uint32_t s_key[2][kS2oMax];
  __shared__ int32_t s_pos[2][kS2oMax];
  __shared__ uint32_t s_cnt[kOrderWaves][256];
  __shared__ uint32_t s_scan[kOrderWaves];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int b, g;
  row_coords(a, row, b, g);
  const int64_t orow = ((int64_t)b * a.Hkv + g) * a.n_cap;
  const int cnt = a.sel_count[(int64_t)b * a.Hkv + g];
  if (cnt <= 1) return;                        // failed (negative), empty or one token
  const int m = min(cnt, kS2oMax);
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
  const int64_t krow = (((int64_t)b * a.Hkv + g) / a.kv_div) * a.n_cap;
  for (int i = tid; i < m; i += kOrderThreads) {
    const int j = a.sel_idx[orow + i];
    IdxRow<T> r;
    r.load(a.k_idx, krow + min(max(j, 0), a.n - 1));
    float l = r.dot(qb) * 0.25f;
    if (l == 0.f) l = 0.f;
    s_key[0][i] = ~order_key(l);               // ascending = logit descending
    s_pos[0][i] = j;
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int cur = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 8 * pass;
    for (int i = tid; i < kOrderWaves * 256; i += kOrderThreads) (&s_cnt[0][0])[i] = 0u;
    __syncthreads();
    uint32_t rank[kOrderRounds], dig[kOrderRounds];
#pragma unroll
    for (int it = 0; it < kOrderRounds; ++it) {
      const int e = wid * (kOrderRounds * 64) + it * 64 + lane;
      const bool v = e < m;
      const uint32_t d = v ? (s_key[cur][e] >> shift) & 255u : 0u;
      uint64_t eq = __ballot(v);                 // lanes holding the same digit
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const uint64_t bb = __ballot((d >> bit) & 1u);
        eq &= ((d >> bit) & 1u) ? bb : ~bb;
      }
      const uint32_t before = s_cnt[wid][d];
      rank[it] = before + (uint32_t)__popcll(eq & lt);
      dig[it] = d;
      // the digit's lowest lane adds the round's count (every lane of the
      // wave has read the old count: one read instruction for all lanes)
      if (v && (eq & lt) == 0ull) s_cnt[wid][d] = before + (uint32_t)__popcll(eq);
    }
    __syncthreads();
    uint32_t tot = 0;
    if (tid < 256) {
      for (int w = 0; w < kOrderWaves; ++w) {
        const uint32_t c = s_cnt[w][tid];
        s_cnt[w][tid] = tot;
        tot += c;
      }
    }
    uint32_t total;
    const uint32_t base = block_exclusive_scan<uint32_t, kOrderThreads>(tid < 256 ? tot : 0u, s_scan, &total);
    if (tid < 256)
      for (int w = 0; w < kOrderWaves; ++w) s_cnt[w][tid] += base;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kOrderRounds; ++it) {
      const int e = wid * (kOrderRounds * 64) + it * 64 + lane;
      if (e < m) {
        const uint32_t dst = s_cnt[wid][dig[it]] + rank[it];
        s_key[cur ^ 1][dst] = s_key[cur][e];
        s_pos[cur ^ 1][dst] = s_pos[cur][e];
      }
    }
    __syncthreads();
    cur ^= 1;
  }
  for (int i = tid; i < m; i += kOrderThreads) a.sel_idx[orow + i] = s_pos[cur][i];
}

hipError_t launch_select_order(const SelectArgs& a, int dtype, hipStream_t s) {
  const int rows = a.B * a.groups.n;
  if (rows == 0) return hipSuccess;
  if (dtype == 0) hipLaunchKernelGGL((select_order_kernel<bf16_t>), dim3(rows), dim3(kOrderThreads), 0, s, a);
  else hipLaunchKernelGGL((select_order_kernel<float>), dim3(rows), dim3(kOrderThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
