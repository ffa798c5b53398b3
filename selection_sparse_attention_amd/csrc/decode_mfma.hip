// Split-KV sparse decode for bf16 caches, with the QK^T of each gathered
// 16-row tile on the matrix cores.
//
// What it computes is the same as the fp32 split kernel (HGA summary, Core
// mechanism item 4: exact softmax attention over the selected tokens; "Full
// Attention Strikes Back" summary, Methodology item 1: sinks + window for
// local heads; S2O summary, Methodology 1: index-guided loading of
// non-contiguous rows): for every query head h of KV group g,
//   o_h = sum_{j in T_g} softmax_j(q_h . k_j / sqrt(d)) v_j .
//
// Work plan: the visible tokens of all (sequence, KV group) pairs are cut into
// items of about `chunk` list entries, with chunk searched so that the items
// of the whole step - however the selected counts are distributed - give
// every workgroup slot of the launch one item.  Every wave derives the same
// plan from the counts (wave reductions, no LDS, no extra launch); workgroup
// b takes item b, and its four waves take the group's 16-token tiles in turn
// with the waves of the group's other items (wave q of W takes tiles q,
// q + W, ...), so that all waves of a group carry the same number of tiles
// and stream through the list together.  Workgroup 0 records each group's
// items for the combine launch.
//
// Layout per wave, one 16-token tile at a time:
//   * lane l gathers token (l % 16): at k-step s the four lanes of a token
//     hold dims 32 s + 8 (l / 16) .. +8, so each load instruction reads 64
//     contiguous bytes of every row, and the registers are exactly the B
//     operand of v_mfma_f32_16x16x32_bf16 (the query fragment in the A operand
//     follows the same dim mapping, one head per row, rows >= G zero).  The product leaves head h's 16 scores in
//     lane group h/4, register h%4 - no cross-lane sum for q.k at all.
//   * the tile max is a 16-lane DPP rotation reduction, broadcast with
//     readlane; probabilities go through a small LDS buffer to every lane.
//   * lane l owns output dims 2(l % (d/2)) .. +1 and, for d = 64, every
//     second token of the tile; it gathers those V pairs with 4-byte loads
//     (one 256-byte row per wave instruction) and accumulates G heads in fp32.
//   * token ids stream from the list three tiles ahead and K/V rows two tiles
//     ahead (three register sets in rotation); every load is unconditional
//     (rows past the end read the group's row 0 and are masked), so each wait
//     is a partial one and two tiles of loads stay in flight.
#include <algorithm>

#include "args.hpp"
#include "common.hpp"

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaThreads = 256;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, false));
}
// max over the 16 lanes of a DPP row (row_ror 8, 4, 2, 1)
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0x128>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x122>(v));
  v = fmaxf(v, dpp_f<0x121>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0x128>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x122>(v);
  v += dpp_f<0x121>(v);
  return v;
}

// ---------------------------------------------------------------- work plan
__device__ __forceinline__ int group_count(const DecodeArgs& a, int bg) {
  const int g = bg % a.Hkv;
  if ((a.local_mask >> g) & 1ull) {
    const int s = min(a.sinks, a.n);
    return s + (a.n - max(s, a.n - a.window));
  }
  return min(max(a.sel_count[bg], 0), a.n);
}

// Wave-wide sum of an int (DPP row reductions, then the four rows).
__device__ __forceinline__ int wave_sum_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);   // row_ror 8
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);   // row_ror 4
  v += __builtin_amdgcn_update_dpp(0, v, 0x122, 0xF, 0xF, false);   // row_ror 2
  v += __builtin_amdgcn_update_dpp(0, v, 0x121, 0xF, 0xF, false);   // row_ror 1
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

constexpr int kPlanPasses = 8;      // groups held in registers: 64 per pass

// The work plan, made by every wave on its own (no LDS, no barrier): lane i
// holds the visible-token counts of groups i, i + 64, ...; the item size is
// the smallest multiple of 16 (at least min_chunk) for which the groups'
// items (group_items each) number at most target_items, so that every
// workgroup slot of the launch gets one item of about the same size.
// Returns the group and split of item `item` (group -1: no such item) and
// the group's item count; with `table`, also writes every group's (first
// item, item count) there.
struct PlanItem { int bg, split, chunk, ns; };

// Items of a group with `count` visible tokens for item size c: the nearest
// whole number of items (at least one), so that every item of every group
// holds about c tokens (a group of 1.03 c is one item, not one plus a sliver).
__device__ __forceinline__ int group_items(int count, int c) {
  return count > 0 ? max(1, (count + c / 2) / c) : 0;
}

__device__ PlanItem plan_item(const DecodeArgs& a, int item, int2* table) {
  const int lane = threadIdx.x & 63;
  const int ng = a.B * a.Hkv;
  const int passes = (ng + 63) / 64;
  int cnt[kPlanPasses];
  int64_t tot = 0;
#pragma unroll
  for (int p = 0; p < kPlanPasses; ++p) {
    const int bg = p * 64 + lane;
    cnt[p] = (p < passes && bg < ng) ? group_count(a, bg) : 0;
  }
#pragma unroll
  for (int p = 0; p < kPlanPasses; ++p)
    if (p < passes) tot += wave_sum_i(cnt[p]);
  // items for a chunk size c (groups beyond the registers: one pass each)
  auto items = [&](int c) __attribute__((always_inline)) -> int64_t {
    int64_t n = 0;
#pragma unroll
    for (int p = 0; p < kPlanPasses; ++p)
      if (p < passes) n += wave_sum_i(group_items(cnt[p], c));
    for (int p = kPlanPasses; p < passes; ++p) {
      const int bg = p * 64 + lane;
      n += wave_sum_i(bg < ng ? group_items(group_count(a, bg), c) : 0);
    }
    return n;
  };
  const int64_t target = a.target_items;
  auto up16 = [](int64_t x) -> int64_t { return (x + 15) / 16 * 16; };
  int64_t lo = up16(max((int64_t)a.min_chunk, (tot + target - 1) / target));
  int64_t hi = lo;
  if (items((int)lo) > target) {
    // at 2 n every non-empty group is one item: the fewest there can be
    hi = up16(max((int64_t)a.min_chunk, 2 * (int64_t)a.n));
    while (lo < hi) {                          // multiples of 16; items(hi) <= target
      const int64_t mid = lo + (hi - lo) / 32 * 16;
      if (items((int)mid) <= target) hi = mid; else lo = mid + 16;
    }
  }
  const int chunk = (int)hi;
  // number the items group by group and find `item`
  PlanItem r{-1, 0, chunk, 0};
  int carry = 0;
  auto number = [&](int p, int c) __attribute__((always_inline)) {
    const int bg = p * 64 + lane;
    const int ns = (bg < ng) ? group_items(c, chunk) : 0;
    const int incl = wave_inclusive_scan(ns);
    const int first = carry + incl - ns;
    if (table && bg < ng) table[bg] = make_int2(first, ns);
    const uint64_t hit = __ballot(bg < ng && item >= first && item < first + ns);
    if (hit) {
      const int l = __ffsll((unsigned long long)hit) - 1;
      r.bg = p * 64 + l;
      r.split = item - __builtin_amdgcn_readlane(first, l);
      r.ns = __builtin_amdgcn_readlane(ns, l);
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
  };
#pragma unroll
  for (int p = 0; p < kPlanPasses; ++p)
    if (p < passes) number(p, cnt[p]);
  for (int p = kPlanPasses; p < passes; ++p) {
    const int bg = p * 64 + lane;
    number(p, bg < ng ? group_count(a, bg) : 0);
  }
  return r;
}

template <int D>
struct Tile {
  static constexpr int KS = D / 32;            // MFMA k-steps
  static constexpr int NCLS = 128 / D;         // token classes for the V pairs
  static constexpr int VT = 16 / NCLS;         // V rows per lane per tile
  bf16x8 k[KS];
  uint32_t v[VT];
  // this lane's K-role token, -1 if none; with head-mask lists the bits
  // 24 + i say whether head 4 (lane / 16) + i of the group has it in its set
  int tok;
};

template <int D, int G>
struct DecodeShared {
  float p[4][16][8];                           // per wave: p[token][head]
  float m[4][8], l[4][8];
  float acc[4][8][D];
};

template <int D, int G, bool LOCAL, bool HM>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, DecodeShared<D, G>& sh, int item,
                                            int bg, int split, int nsg) {
  using TL = Tile<D>;
  constexpr int KS = TL::KS, NCLS = TL::NCLS, VT = TL::VT;
  static_assert(G <= 8, "at most 8 query heads per KV group");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int n = a.n;
  int s_eff = 0, wst = 0, count;
  if (LOCAL) {
    s_eff = min(a.sinks, n);
    wst = max(s_eff, n - a.window);
    count = s_eff + (n - wst);
  } else {
    count = min(max(a.sel_count[bg], 0), n);
  }
  const int64_t row0 = (int64_t)bg * a.n_cap;          // the group's list
  const int64_t kv0 = (int64_t)(bg / a.kv_div) * a.n_cap;   // its K/V rows

  // query fragment: head (lane % 16), this lane's slice of the k mapping
  bf16x8 qf[KS];
  {
    const int h = lane & 15, jq = lane >> 4;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (h < G) {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                             ((int64_t)b * a.Hq + g * G + h) * D + 32 * s + 8 * jq;
        w = *reinterpret_cast<const u32x4*>(qp);
      }
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // this wave's contiguous share of the item, in whole 16-token tiles
  // the group's waves take its tiles in turn (tile q, q + W, ...)
  const int Wg = 4 * nsg, qw = 4 * split + wid;
  const int Tg = (count + 15) / 16;
  const int ntiles = (Tg > qw) ? (Tg - qw + Wg - 1) / Wg : 0;

  const int kt = lane & 15, jg = lane >> 4;            // K role
  const int vd = 2 * (lane % (D / 2)), vc = lane / (D / 2);   // V role
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + kv0 * D + 8 * jg;
  // V rows: a wave-uniform row address (scalar) plus this lane's dims
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + kv0 * D;

  // raw list entry of this lane's token in a tile (a load for listed groups,
  // in bounds even past the end; checked when it is used)
  auto raw_id = [&](int tile) __attribute__((always_inline)) -> int {
    const int e = (qw + tile * Wg) * 16 + kt;
    if (LOCAL) return (e < s_eff) ? e : wst + (e - s_eff);
    return a.sel_idx[row0 + min(e, count - 1)];
  };
  // issue a tile's K and V loads
  auto issue = [&](int tile, TL& t, int raw) __attribute__((always_inline)) {
    const int e = (qw + tile * Wg) * 16 + kt;
    // head-mask lists: the position is the low 24 bits, the heads the top 8
    const int pos = HM ? (raw & 0xFFFFFF) : raw;
    const int tok = (e < count && (unsigned)pos < (unsigned)n)
                        ? (HM ? pos | (int)((((uint32_t)raw >> 24 >> (4 * jg)) & 0xFu) << 24) : pos)
                        : -1;
    t.tok = tok;
    const uint16_t* kp = kbase + (int64_t)(HM ? max(tok, 0) & 0xFFFFFF : max(tok, 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      t.k[s] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + 32 * s)));
#pragma unroll
    for (int r = 0; r < VT; ++r) {
      int tv = __builtin_amdgcn_readlane(tok, r * NCLS);
      if (NCLS == 2) {
        const int tv1 = __builtin_amdgcn_readlane(tok, r * NCLS + 1);
        tv = vc ? tv1 : tv;
      }
      const uint16_t* vrow = vbase + (int64_t)(HM ? max(tv, 0) & 0xFFFFFF : max(tv, 0)) * D;
      t.v[r] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vrow + vd));
    }
  };

  float m[G], lsum[4], acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; acc[h][0] = 0.f; acc[h][1] = 0.f; }
#pragma unroll
  for (int i = 0; i < 4; ++i) lsum[i] = 0.f;
  const float sc = a.scale_log2;

  auto compute = [&](const TL& t) __attribute__((always_inline)) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[s], t.k[s], c, 0, 0, 0);
    const bool valid = t.tok >= 0;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // lane group jg holds heads 4 jg .. 4 jg + 3 of its token
      const bool mine = !HM || ((t.tok >> (24 + i)) & 1);
      sv[i] = (valid && mine) ? c[i] * sc : -INFINITY;
    }
    float alpha[G];
    bool moved = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int grp = h >> 2, r = h & 3;
      const float tm = row16_max(sv[r]);
      const float tmax =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tm), 16 * grp));
      const float mn = fmaxf(m[h], tmax);
      alpha[h] = (m[h] == mn) ? 1.f : exp2f(m[h] - mn);
      moved |= (m[h] != mn);
      m[h] = mn;
      if (jg == grp) {
        const float p = (sv[r] == -INFINITY) ? 0.f : exp2f(sv[r] - mn);
        lsum[r] = lsum[r] * alpha[h] + p;
        sh.p[wid][kt][h] = p;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (moved) {                                 // wave-uniform: m is uniform
#pragma unroll
      for (int h = 0; h < G; ++h) { acc[h][0] *= alpha[h]; acc[h][1] *= alpha[h]; }
    }
#pragma unroll
    for (int r = 0; r < VT; ++r) {
      const int tt = r * NCLS + vc;
      const float v0 = bf16_lo(t.v[r]), v1 = bf16_hi(t.v[r]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = sh.p[wid][tt][h];
        acc[h][0] = fmaf(p, v0, acc[h][0]);
        acc[h][1] = fmaf(p, v1, acc[h][1]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  if (ntiles > 0) {
    TL ta, tb, tc;
    const int r0 = raw_id(0);
    const int r1 = raw_id(1);
    issue(0, ta, r0);
    issue(1, tb, r1);
    int rawp = raw_id(2);
    // one step: ids of tile t+3 requested, rows of tile t+2 issued, tile t
    // computed
    auto step = [&](int tl, TL& cur, TL& ahead2) __attribute__((always_inline)) {
      const int rn = raw_id(tl + 3);
      issue(tl + 2, ahead2, rawp);
      rawp = rn;
      compute(cur);
    };
    int t = 0;
    for (; t + 2 < ntiles; t += 3) {
      step(t, ta, tc);
      step(t + 1, tb, ta);
      step(t + 2, tc, tb);
    }
    if (t < ntiles) step(t, ta, tc);
    if (t + 1 < ntiles) step(t + 1, tb, ta);
  }

  // wave result: l from the lanes of each head's group, acc from all lanes
  // (for d = 64 the two token classes hold the same dims: add them)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (NCLS == 2) {
      acc[h][0] += __shfl_xor(acc[h][0], 32);
      acc[h][1] += __shfl_xor(acc[h][1], 32);
    }
  }
  float lw[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int grp = h >> 2, r = h & 3;
    const float ls = row16_sum(lsum[r]);
    lw[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls), 16 * grp));
  }
  if (lane < D / 2) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sh.acc[wid][h][vd] = acc[h][0];
      sh.acc[wid][h][vd + 1] = acc[h][1];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sh.m[wid][h] = (ntiles > 0) ? m[h] : -INFINITY;
      sh.l[wid][h] = (ntiles > 0) ? lw[h] : 0.f;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kMfmaThreads) {
    const int h = idx / D, e = idx % D;
    float M = sh.m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sh.m[w][h]);
    float av = 0.f, lv = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sh.m[w][h];
      const float wt = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      av += wt * sh.acc[w][h][e];
      lv += wt * sh.l[w][h];
    }
    float* pp = a.partial + ((int64_t)item * G + h) * (D + 2);
    pp[e] = av;
    if (e == 0) { pp[D] = M; pp[D + 1] = lv; }
  }
}

template <int D, int G, bool HM>
__global__ __launch_bounds__(kMfmaThreads, (G > 4 ? 1 : 2)) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ DecodeShared<D, G> sh;
  // every wave makes the same plan; wave 0 of workgroup 0 also records every
  // group's items for the combine launch
  const PlanItem pl = plan_item(a, blockIdx.x, (blockIdx.x == 0 && threadIdx.x < 64) ? a.plan : nullptr);
  const int bg = pl.bg, split = pl.split, nsg = pl.ns;
  if (bg < 0) return;
  if ((a.local_mask >> (bg % a.Hkv)) & 1ull) decode_item<D, G, true, false>(a, sh, blockIdx.x, bg, split, nsg);
  else decode_item<D, G, false, HM>(a, sh, blockIdx.x, bg, split, nsg);
}

// Merge the items of one (sequence, query head).  Thread (e, part) owns
// output dim e for a share of the items; per round of P x CH items every
// thread issues all its acc loads and the m / l loads at once (one memory
// latency per round), the round's m / l go through LDS, and the (M, L, A)
// state is merged online across rounds.  The head's item range comes from
// the table the decode launch wrote.
template <int D, int G>
__global__ __launch_bounds__(kMfmaThreads) void decode_item_combine_kernel(DecodeArgs a) {
  constexpr int P = kMfmaThreads / D;          // item shares per output dim
  constexpr int CH = 16;                       // items per thread per round
  constexpr int R = P * CH;                    // items per round
  __shared__ float s_m[R], s_l[R];
  __shared__ float s_a[kMfmaThreads];
  const int bgh = blockIdx.x;
  const int bg = bgh / G, h = bgh - bg * G;
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int2 fr = a.plan[bg];
  const int first = fr.x, ns = fr.y;
  const int tid = threadIdx.x, e = tid % D, part = tid / D;
  const int64_t stride = (int64_t)G * (D + 2);
  const float* base = a.partial + ((int64_t)first * G + h) * (D + 2);
  float M = -INFINITY, L = 0.f, A = 0.f;
  for (int c0 = 0; c0 < ns; c0 += R) {
    float av[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int i = c0 + part * CH + j;
      const float x = base[min(i, ns - 1) * stride + e];
      av[j] = (i < ns) ? x : 0.f;
    }
    if (tid < R) {
      const int i = c0 + tid;
      const float* q = base + min(i, ns - 1) * stride;
      const float mi = q[D], li = q[D + 1];
      s_m[tid] = (i < ns) ? mi : -INFINITY;
      s_l[tid] = (i < ns) ? li : 0.f;
    }
    __syncthreads();
    float Mr = -INFINITY;
#pragma unroll
    for (int j = 0; j < R; ++j) Mr = fmaxf(Mr, s_m[j]);
    const float Mn = fmaxf(M, Mr);
    if (Mn != -INFINITY) {
      const float sc = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
      A *= sc;
      L *= sc;
      float Lr = 0.f;
#pragma unroll
      for (int j = 0; j < R; ++j) Lr = fmaf(exp2f(s_m[j] - Mn), s_l[j], Lr);   // 0 for m = -inf
      L += Lr;
#pragma unroll
      for (int j = 0; j < CH; ++j) A = fmaf(exp2f(s_m[part * CH + j] - Mn), av[j], A);
      M = Mn;
    }
    __syncthreads();
  }
  s_a[tid] = A;
  __syncthreads();
  if (part == 0) {
    float v = A;
#pragma unroll
    for (int q = 1; q < P; ++q) v += s_a[q * D + e];
    if ((a.s2o_mask >> g) & 1ull) {
      // an early-stop group's first pass: its state, for the early-stop kernel
      float* st = a.s2o_state + (bg * G + h) * (D + 2);
      st[e] = v;
      if (e == 0) { st[D] = M; st[D + 1] = L; }
      return;
    }
    // a failed selection (negative count) poisons the group's outputs (the
    // head's own, with head-mask lists)
    const bool failed = !((a.local_mask >> g) & 1ull) &&
                        (a.head_masks ? a.head_count[(int64_t)b * a.Hq + g * G + h] < 0 : a.sel_count[bg] < 0);
    a.out[((int64_t)b * a.Hq + g * G + h) * D + e] = failed ? __builtin_nanf("") : ((L > 0.f) ? v / L : 0.f);
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int d, hipStream_t s) {
  if (a.max_splits < 1 || a.target_items < 1 || !a.plan) return hipErrorInvalidValue;
  dim3 grid(a.max_splits), block(kMfmaThreads);
#define SA_DEC(D_, G_)                                                                         \
  do {                                                                                         \
    if (a.head_masks) hipLaunchKernelGGL((decode_mfma_kernel<D_, G_, true>), grid, block, 0, s, a); \
    else hipLaunchKernelGGL((decode_mfma_kernel<D_, G_, false>), grid, block, 0, s, a);        \
  } while (0)
  if (d == 128) {
    switch (a.G) {
      case 1: SA_DEC(128, 1); break;
      case 2: SA_DEC(128, 2); break;
      case 4: SA_DEC(128, 4); break;
      case 8: SA_DEC(128, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else if (d == 64) {
    switch (a.G) {
      case 1: SA_DEC(64, 1); break;
      case 2: SA_DEC(64, 2); break;
      case 4: SA_DEC(64, 4); break;
      case 8: SA_DEC(64, 8); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef SA_DEC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid(a.B * a.Hq);
#define SA_CMB(D_, G_) hipLaunchKernelGGL((decode_item_combine_kernel<D_, G_>), cgrid, block, 0, s, a)
  switch (a.G * 1000 + d) {
    case 1128: SA_CMB(128, 1); break;
    case 2128: SA_CMB(128, 2); break;
    case 4128: SA_CMB(128, 4); break;
    case 8128: SA_CMB(128, 8); break;
    case 1064: SA_CMB(64, 1); break;
    case 2064: SA_CMB(64, 2); break;
    case 4064: SA_CMB(64, 4); break;
    case 8064: SA_CMB(64, 8); break;
    default: return hipErrorInvalidValue;
  }
#undef SA_CMB
  return hipGetLastError();
}

// ---------------------------------------------------------------- head union
// Per-head sets decoded per KV group: the union of the G heads' sets of one
// (sequence, selecting group), each position tagged with the heads that
// chose it, so that the decode gathers every row once for all G heads and
// masks each head's scores to its own set.  The positions are cut into
// slices of kUnionSlice; two launches spread over the whole chip:
//   1. per (slice, group, sequence): each head's entries inside the slice
//      (its list is ascending: one wave per head finds the slice's first
//      and last entries with 64-way searches, three dependent loads for a
//      32K list) set their head bits in an LDS byte per position; the
//      slice's bytes and its count of tagged positions go to the workspace;
//   2. per (slice, group, sequence): the slice's entries (head bits << 24 |
//      position) written in order at the sum of the earlier slices' counts.
constexpr int kUnionThreads = 256;

// First index i in [lo, hi) of the ascending list with x[i] >= v (hi if
// none); one wave, every lane returns it.  64-way: each round reads 64
// evenly spaced entries and keeps the sub-range where the bound lies.
__device__ __forceinline__ int wave_lower_bound(const int32_t* x, int lo, int hi, int v) {
  const int lane = threadIdx.x & 63;
  while (hi - lo > 64) {
    const int64_t span = hi - lo;
    const int probe = lo + (int)((span * lane) / 64);          // lane 0 probes lo
    const bool below = x[probe] < v;
    const uint64_t m = __ballot(below);
    const int k = __popcll(m);                                  // probes below v (a prefix)
    const int nlo = (k == 0) ? lo : lo + (int)((span * (k - 1)) / 64);
    const int nhi = (k == 64) ? hi : lo + (int)((span * k) / 64) + 1;
    lo = nlo;
    hi = min(hi, nhi);
  }
  const int i = lo + lane;
  const bool below = i < hi && x[i] < v;
  return lo + __popcll(__ballot(below));
}

// grid (slice, group, sequence)
__global__ __launch_bounds__(kUnionThreads) void head_union_mark_kernel(HeadUnionArgs a) {
  __shared__ uint32_t s_hm[kUnionSlice / 4];
  __shared__ int s_lo[8], s_hi[8];
  __shared__ int32_t s_red[kUnionThreads / 64];
  const int g = a.groups.ids[blockIdx.y], b = blockIdx.z, tid = threadIdx.x;
  const int wid = tid >> 6, lane = tid & 63;
  const int p0 = blockIdx.x * kUnionSlice, p1 = min(a.n, p0 + kUnionSlice);
  for (int i = tid; i < kUnionSlice / 4; i += kUnionThreads) s_hm[i] = 0u;
  // each head's entries inside [p0, p1)
  for (int h = wid; h < a.G; h += kUnionThreads / 64) {
    const int64_t row = (int64_t)b * a.Hq + g * a.G + h;
    const int cnt = min(max(a.sel_count[row], 0), a.n);
    const int32_t* lst = a.sel_idx + row * a.n_cap;
    const int lo = wave_lower_bound(lst, 0, cnt, p0);
    const int hi = wave_lower_bound(lst, lo, cnt, p1);
    if (lane == 0) { s_lo[h] = lo; s_hi[h] = hi; }
  }
  __syncthreads();
  for (int h = 0; h < a.G; ++h) {
    const int32_t* lst = a.sel_idx + ((int64_t)b * a.Hq + g * a.G + h) * a.n_cap;
    const int lo = s_lo[h], hi = s_hi[h];
    for (int i = lo + tid; i < hi; i += kUnionThreads) {
      const int q = lst[i] - p0;
      if ((unsigned)q < (unsigned)(p1 - p0)) atomicOr(&s_hm[q >> 2], (1u << h) << (8 * (q & 3)));
    }
  }
  __syncthreads();
  uint32_t* out = a.masks + ((int64_t)b * a.Hkv + g) * a.mask_words + p0 / 4;
  int c = 0;
  for (int w = tid; w < (p1 - p0 + 3) / 4; w += kUnionThreads) {
    const uint32_t x = s_hm[w];
    out[w] = x;
    c += ((x & 0xFFu) != 0) + ((x & 0xFF00u) != 0) + ((x & 0xFF0000u) != 0) + ((x >> 24) != 0);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) c += __shfl_xor(c, o);
  if (lane == 0) s_red[wid] = c;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int w = 0; w < kUnionThreads / 64; ++w) t += s_red[w];
    a.slice_count[((int64_t)b * a.Hkv + g) * a.n_slices + blockIdx.x] = t;
  }
}

// grid (slice, group, sequence)
__global__ __launch_bounds__(kUnionThreads) void head_union_compact_kernel(HeadUnionArgs a) {
  __shared__ int32_t s_scan[kUnionThreads / 64];
  const int g = a.groups.ids[blockIdx.y], b = blockIdx.z, tid = threadIdx.x;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const int p0 = blockIdx.x * kUnionSlice, p1 = min(a.n, p0 + kUnionSlice);
  const int32_t* cnts = a.slice_count + bg * a.n_slices;
  int before = 0;
  for (int s = 0; s < blockIdx.x; ++s) before += cnts[s];
  // thread t: 2 consecutive words (8 positions) of the slice
  constexpr int PW = kUnionSlice / 4 / kUnionThreads;
  const uint32_t* m = a.masks + bg * a.mask_words + p0 / 4;
  const int nw = (p1 - p0 + 3) / 4;
  uint32_t x[PW];
  int mine = 0;
#pragma unroll
  for (int k = 0; k < PW; ++k) {
    const int w = tid * PW + k;
    x[k] = (w < nw) ? m[w] : 0u;
    mine += ((x[k] & 0xFFu) != 0) + ((x[k] & 0xFF00u) != 0) + ((x[k] & 0xFF0000u) != 0) + ((x[k] >> 24) != 0);
  }
  int32_t total;
  int32_t o = before + block_exclusive_scan<int32_t, kUnionThreads>(mine, s_scan, &total);
  int32_t* out = a.union_idx + bg * a.n_cap;
#pragma unroll
  for (int k = 0; k < PW; ++k) {
    const int w = tid * PW + k;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t hm = (x[k] >> (8 * q)) & 0xFFu;
      if (hm) out[o++] = (int32_t)((hm << 24) | (uint32_t)(p0 + 4 * w + q));
    }
  }
  if (tid == 0 && blockIdx.x == a.n_slices - 1) a.union_count[bg] = before + total;
}

hipError_t launch_head_union(const HeadUnionArgs& a, hipStream_t s) {
  if (a.G < 1 || a.G > 8 || a.n < 1 || a.n > kUnionMaxN || a.n_cap < a.n) return hipErrorInvalidValue;
  if (a.mask_words != (a.n + 3) / 4 || a.n_slices != (a.n + kUnionSlice - 1) / kUnionSlice)
    return hipErrorInvalidValue;
  if (a.groups.n == 0 || a.B == 0) return hipSuccess;
  const dim3 grid(a.n_slices, a.groups.n, a.B);
  hipLaunchKernelGGL(head_union_mark_kernel, grid, dim3(kUnionThreads), 0, s, a);
  hipLaunchKernelGGL(head_union_compact_kernel, grid, dim3(kUnionThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- early stop
// Monotone-gain early stop ("S2O" summary, Methodology 2-3) for the groups in
// a.s2o, whose lists hold their top-k candidates in visit order (index logit
// descending).  One 512-thread workgroup per (group, sequence), the group's
// G heads in one MFMA tile as above; blocks of 64 tokens go in rounds of
// two, wave w taking tile w % 4 of block w / 4 of the round:
//   * first pass: the local rule's tokens (sinks + window), computed by the
//     split kernels (all groups at once) and resumed here from the cached
//     (m, l, acc) of each head - the page's two-pass structure;
//   * the candidates outside the first pass, staged in LDS in visit order
//     (each wave compacts an eighth of the list with ballots);
//   * after scoring a round of candidate blocks, the waves exchange through
//     LDS, per head, each tile's (max, sum) and their state before the round
//     (double-buffered: one barrier per round); every wave then takes the
//     same decisions block by block in order: S_blk, the block's mass, and
//     S_before, the mass attended before it; the head stops at the first
//     block with S_blk < tau * S_before (that block is kept) - exactly the
//     block-by-block rule; stopped heads take no more tokens, and the group
//     ends when every head has stopped;
//   * the next round's rows are requested before the current round is
//     scored.
// Outputs go straight to `out` (the whole group is one workgroup).
constexpr int kS2oThreads = 512;
constexpr int kS2oWaves = kS2oThreads / 64;
constexpr int kRound = kS2oWaves / 4;            // blocks per round

template <int D>
struct S2oShared {
  float p[kS2oWaves][16][8];                     // per wave: p[token][head]
  float m[kS2oWaves][8], l[kS2oWaves][8];
  float acc[kS2oWaves][8][D];
  int visit[kS2oMax];
  float tm[2][kRound][4][8], ts[2][kRound][4][8];   // [parity][block][tile][head]
  float sm[2][kS2oWaves][8], sl[2][kS2oWaves][8];  // [parity][wave][head]
  int cnt[kS2oWaves];
};

template <int D, int G>
__global__ __launch_bounds__(kS2oThreads) void decode_s2o_kernel(DecodeArgs a) {
  using TL = Tile<D>;
  constexpr int KS = TL::KS, NCLS = TL::NCLS, VT = TL::VT;
  static_assert(G <= 8, "at most 8 query heads per KV group");
  __shared__ S2oShared<D> sh;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int br = wid >> 2, tw = wid & 3;          // this wave's block of a round, and tile of it
  const int b = blockIdx.y, g = a.s2o.ids[blockIdx.x];
  const int bg = b * a.Hkv + g;
  const int n = a.n;
  const int s_eff = min(a.sinks, n), wst = max(s_eff, n - a.window);
  const int c0 = s_eff + (n - wst);                         // first-pass tokens
  const int raw_count = a.sel_count[bg];
  const int count = min(max(raw_count, 0), min(n, kS2oMax));
  const int64_t row0 = (int64_t)bg * a.n_cap;
  const int64_t kv0 = (int64_t)(bg / a.kv_div) * a.n_cap;

  // ---- the visit list: candidates outside the first pass, in list order
  {
    const int Q = (count + kS2oWaves - 1) / kS2oWaves;
    const int lo = min(count, wid * Q), hi = min(count, lo + Q);
    int kept = 0;
    for (int base = lo; base < hi; base += 64) {
      const int e = base + lane;
      const int j = (e < hi) ? a.sel_idx[row0 + e] : -1;
      const bool keep = e < hi && (unsigned)j < (unsigned)n && !(j < s_eff || j >= wst);
      kept += __popcll(__ballot(keep));
    }
    if (lane == 0) sh.cnt[wid] = kept;
    __syncthreads();
    int run = 0;
    for (int w = 0; w < wid; ++w) run += sh.cnt[w];
    for (int base = lo; base < hi; base += 64) {
      const int e = base + lane;
      const int j = (e < hi) ? a.sel_idx[row0 + e] : -1;
      const bool keep = e < hi && (unsigned)j < (unsigned)n && !(j < s_eff || j >= wst);
      const uint64_t bal = __ballot(keep);
      if (keep) sh.visit[run + __popcll(bal & ((1ull << lane) - 1ull))] = j;
      run += __popcll(bal);
    }
  }
  __syncthreads();
  int nv = 0;
  for (int w = 0; w < kS2oWaves; ++w) nv += sh.cnt[w];
  (void)c0;
  const int nb0 = 0, nbt = (nv + 63) / 64;       // the first pass is resumed, not recomputed

  // query fragment: head (lane % 16), this lane's slice of the k mapping
  bf16x8 qf[KS];
  {
    const int h = lane & 15, jq = lane >> 4;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (h < G) {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                             ((int64_t)b * a.Hq + g * G + h) * D + 32 * s + 8 * jq;
        w = *reinterpret_cast<const u32x4*>(qp);
      }
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }
  const int kt = lane & 15, jg = lane >> 4;
  const int vd = 2 * (lane % (D / 2)), vc = lane / (D / 2);
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + kv0 * D + 8 * jg;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + kv0 * D;
  // this lane's token of block blk (this wave's tile of it), -1 if none
  auto token = [&](int blk) __attribute__((always_inline)) -> int {
    if (blk >= nbt) return -1;
    const int e = 64 * blk + 16 * tw + kt;
    if (blk < nb0) return (e < c0) ? ((e < s_eff) ? e : wst + (e - s_eff)) : -1;
    const int ev = e - 64 * nb0;
    return (ev < nv) ? sh.visit[ev] : -1;
  };
  auto issue = [&](int blk, TL& t) __attribute__((always_inline)) {
    const int tok = token(blk);
    t.tok = tok;
    const uint16_t* kp = kbase + (int64_t)max(tok, 0) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      t.k[s] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + 32 * s)));
#pragma unroll
    for (int r = 0; r < VT; ++r) {
      int tv = __builtin_amdgcn_readlane(tok, r * NCLS);
      if (NCLS == 2) {
        const int tv1 = __builtin_amdgcn_readlane(tok, r * NCLS + 1);
        tv = vc ? tv1 : tv;
      }
      const uint16_t* vrow = vbase + (int64_t)max(tv, 0) * D;
      t.v[r] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vrow + vd));
    }
  };

  float m[G], lsum[4], acc[G][2];
  bool active[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; acc[h][0] = 0.f; acc[h][1] = 0.f; active[h] = true; }
#pragma unroll
  for (int i = 0; i < 4; ++i) lsum[i] = 0.f;
  if (wid == 0) {
    // wave 0 starts from the first pass: m everywhere, l on the first lane of
    // the head's lane group, acc on the lanes that own the dims
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float* st = a.s2o_state + ((int64_t)bg * G + h) * (D + 2);
      m[h] = st[D];
      if (jg == (h >> 2) && kt == 0) lsum[h & 3] = st[D + 1];
      if (vc == 0) { acc[h][0] = st[vd]; acc[h][1] = st[vd + 1]; }
    }
  }
  const float sc = a.scale_log2;
  const float tau = a.s2o_tau;

  // one round: blocks blk0 .. blk0 + nr - 1 (never mixing the first pass with
  // candidates); this wave holds tile tw of block blk0 + br
  auto round_step = [&](int blk0, int nr, int rnd, const TL& t) __attribute__((always_inline)) -> bool {
    const bool cand = blk0 >= nb0;
    float sv[4];
    {
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[s], t.k[s], c, 0, 0, 0);
      const bool valid = br < nr && t.tok >= 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = valid ? c[i] * sc : -INFINITY;
    }
    int keep[G];                                   // last block of the round each head keeps
#pragma unroll
    for (int h = 0; h < G; ++h) keep[h] = active[h] ? kRound - 1 : -1;
    if (cand) {
      const int par = rnd & 1;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const int grp = h >> 2, ri = h & 3;
        const float tm = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, row16_max(sv[ri])), 16 * grp));
        const float e = (tm == -INFINITY || sv[ri] == -INFINITY) ? 0.f : exp2f(sv[ri] - tm);
        const float ts = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, row16_sum(e)), 16 * grp));
        const float lw = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, row16_sum(lsum[ri])), 16 * grp));
        if (lane == 0) {
          sh.tm[par][br][tw][h] = tm;
          sh.ts[par][br][tw][h] = ts;
          sh.sm[par][wid][h] = m[h];
          sh.sl[par][wid][h] = lw;
        }
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // mass before the round, (mp, sp): sp relative to mp
        float mp = -INFINITY;
        for (int w = 0; w < kS2oWaves; ++w) mp = fmaxf(mp, sh.sm[par][w][h]);
        float sp = 0.f;
        for (int w = 0; w < kS2oWaves; ++w)
          if (sh.sl[par][w][h] > 0.f) sp += sh.sl[par][w][h] * exp2f(sh.sm[par][w][h] - mp);
        bool act = active[h];
        int kp = act ? nr - 1 : -1;
        for (int r = 0; r < nr && act; ++r) {
          float mb = -INFINITY;
#pragma unroll
          for (int q = 0; q < 4; ++q) mb = fmaxf(mb, sh.tm[par][r][q][h]);
          float sb = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (sh.ts[par][r][q][h] > 0.f) sb += sh.ts[par][r][q][h] * exp2f(sh.tm[par][r][q][h] - mb);
          const float ref = fmaxf(mb, mp);
          const float gain = (sb > 0.f) ? sb * exp2f(mb - ref) : 0.f;
          const float before = (sp > 0.f) ? sp * exp2f(mp - ref) : 0.f;
          if (before > 0.f && gain < tau * before) { kp = r; act = false; break; }
          sp = before + gain;                      // the block joins the mass before the next
          mp = ref;
        }
        keep[h] = kp;
        active[h] = act;
      }
    }
    // merge this wave's tile, head h if its block is kept
    float alpha[G];
    bool moved = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int grp = h >> 2, ri = h & 3;
      const bool take = br < nr && br <= keep[h];
      const float tmx = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, row16_max(sv[ri])), 16 * grp));
      const float mn = take ? fmaxf(m[h], tmx) : m[h];
      alpha[h] = (m[h] == mn) ? 1.f : exp2f(m[h] - mn);
      moved |= (m[h] != mn);
      m[h] = mn;
      if (jg == grp) {
        const float p = (!take || sv[ri] == -INFINITY) ? 0.f : exp2f(sv[ri] - mn);
        lsum[ri] = lsum[ri] * alpha[h] + p;
        sh.p[wid][kt][h] = p;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (moved) {
#pragma unroll
      for (int h = 0; h < G; ++h) { acc[h][0] *= alpha[h]; acc[h][1] *= alpha[h]; }
    }
#pragma unroll
    for (int q = 0; q < VT; ++q) {
      const int tt = q * NCLS + vc;
      const float v0 = bf16_lo(t.v[q]), v1 = bf16_hi(t.v[q]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = sh.p[wid][tt][h];
        acc[h][0] = fmaf(p, v0, acc[h][0]);
        acc[h][1] = fmaf(p, v1, acc[h][1]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    bool any = false;
#pragma unroll
    for (int h = 0; h < G; ++h) any |= active[h];
    return any;
  };

  if (raw_count >= 0) {
    // rounds of up to kRound blocks: the first pass, then the candidates (a
    // round never mixes the two); the next round's rows are requested
    // before the current one is scored
    auto round_len = [&](int blk) __attribute__((always_inline)) {
      return min(kRound, ((blk < nb0) ? nb0 : nbt) - blk);
    };
    TL ta, tb;
    int blk = 0, rnd = 0;
    int nr = round_len(0);
    issue(br < nr ? br : nbt, ta);
    while (blk < nbt) {
      const int nblk = blk + nr, nnr = (nblk < nbt) ? round_len(nblk) : 0;
      issue(br < nnr ? nblk + br : nbt, tb);
      if (!round_step(blk, nr, rnd, ta)) break;
      blk = nblk; nr = nnr; ++rnd;
      if (blk >= nbt) break;
      const int nblk2 = blk + nr, nnr2 = (nblk2 < nbt) ? round_len(nblk2) : 0;
      issue(br < nnr2 ? nblk2 + br : nbt, ta);
      if (!round_step(blk, nr, rnd, tb)) break;
      blk = nblk2; nr = nnr2; ++rnd;
    }
  }

  // merge the waves and write the group's outputs
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (NCLS == 2) {
      acc[h][0] += __shfl_xor(acc[h][0], 32);
      acc[h][1] += __shfl_xor(acc[h][1], 32);
    }
  }
  float lw[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int grp = h >> 2, ri = h & 3;
    const float ls = row16_sum(lsum[ri]);
    lw[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ls), 16 * grp));
  }
  __syncthreads();
  if (lane < D / 2) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sh.acc[wid][h][vd] = acc[h][0];
      sh.acc[wid][h][vd + 1] = acc[h][1];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { sh.m[wid][h] = m[h]; sh.l[wid][h] = lw[h]; }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kS2oThreads) {
    const int h = idx / D, e = idx % D;
    float M = sh.m[0][h];
    for (int w = 1; w < kS2oWaves; ++w) M = fmaxf(M, sh.m[w][h]);
    float av = 0.f, lv = 0.f;
    for (int w = 0; w < kS2oWaves; ++w) {
      const float mw = sh.m[w][h];
      const float wt = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      av += wt * sh.acc[w][h][e];
      lv += wt * sh.l[w][h];
    }
    a.out[((int64_t)b * a.Hq + g * G + h) * D + e] =
        (raw_count < 0) ? __builtin_nanf("") : ((lv > 0.f) ? av / lv : 0.f);
  }
}

hipError_t launch_decode_s2o(const DecodeArgs& a, int d, hipStream_t s) {
  if (a.s2o.n == 0) return hipSuccess;
  dim3 grid(a.s2o.n, a.B), block(kS2oThreads);
#define SA_S2O(D_, G_) hipLaunchKernelGGL((decode_s2o_kernel<D_, G_>), grid, block, 0, s, a)
  switch (a.G * 1000 + d) {
    case 1128: SA_S2O(128, 1); break;
    case 2128: SA_S2O(128, 2); break;
    case 4128: SA_S2O(128, 4); break;
    case 8128: SA_S2O(128, 8); break;
    case 1064: SA_S2O(64, 1); break;
    case 2064: SA_S2O(64, 2); break;
    case 4064: SA_S2O(64, 4); break;
    case 8064: SA_S2O(64, 8); break;
    default: return hipErrorInvalidValue;
  }
#undef SA_S2O
  return hipGetLastError();
}

}  // namespace sa
