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
// items of `chunk` consecutive list entries, with chunk = total / target
// (rounded up to 64), so that the items of the whole step - however the
// selected counts are distributed - fill the chip about once.  Every
// workgroup derives the same plan from the counts (a block reduction and a
// scan over the groups, no extra launch) and takes item blockIdx.x; the
// combine launch re-derives it to find each head's items.
//
// Layout per wave, one 16-token tile at a time:
//   * lane l gathers d/4 consecutive K elements of token (l % 16): the four
//     lanes of a token cover its row, and they are exactly the B operand of
//     v_mfma_f32_16x16x32_bf16 (k-step s uses elements 8s..8s+7 of each lane's
//     slice; the query fragment in the A operand follows the same mapping, one
//     head per row, rows >= G zero).  The product leaves head h's 16 scores in
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
#include "args.hpp"
#include "common.hpp"

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaThreads = 256;
constexpr int kMaxItemsLds = 8192;           // items one combine workgroup merges

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

// The item size: all visible tokens over target_items items, rounded up to
// 64 entries, at least min_chunk.  Identical in every workgroup.
__device__ int plan_chunk(const DecodeArgs& a, int64_t* s_scan) {
  int64_t t = 0;
  for (int bg = threadIdx.x; bg < a.B * a.Hkv; bg += kMfmaThreads) t += group_count(a, bg);
  int64_t tot;
  (void)block_exclusive_scan<int64_t, kMfmaThreads>(t, s_scan, &tot);
  int64_t c = (tot + a.target_items - 1) / a.target_items;
  c = (c + 63) / 64 * 64;
  return (int)(c > a.min_chunk ? c : a.min_chunk);
}

// Number the items group by group (ceil(count / chunk) each).  Leaves in
// s_out: [0] the group of item `item` (-1 when the plan has fewer items),
// [1] its split within the group, [2] the first item of group `want`, [3]
// that group's item count.
__device__ void plan_walk(const DecodeArgs& a, int chunk, int item, int want, int* s_scan,
                          int* s_out) {
  if (threadIdx.x == 0) { s_out[0] = -1; s_out[1] = 0; s_out[2] = 0; s_out[3] = 0; }
  __syncthreads();
  const int ng = a.B * a.Hkv;
  int carry = 0;
  for (int base = 0; base < ng; base += kMfmaThreads) {
    const int bg = base + threadIdx.x;
    const int ns = (bg < ng) ? (group_count(a, bg) + chunk - 1) / chunk : 0;
    int tot;
    const int first = carry + block_exclusive_scan<int, kMfmaThreads>(ns, s_scan, &tot);
    if (bg < ng) {
      if (item >= first && item < first + ns) { s_out[0] = bg; s_out[1] = item - first; }
      if (bg == want) { s_out[2] = first; s_out[3] = ns; }
    }
    carry += tot;
  }
  __syncthreads();
}

template <int D>
struct Tile {
  static constexpr int KS = D / 32;            // MFMA k-steps
  static constexpr int NCLS = 128 / D;         // token classes for the V pairs
  static constexpr int VT = 16 / NCLS;         // V rows per lane per tile
  bf16x8 k[KS];
  uint32_t v[VT];
  int tok;                                     // this lane's K-role token, -1 if none
};

template <int D, int G>
struct DecodeShared {
  int64_t scan64[kMfmaThreads / 64];
  int scan32[kMfmaThreads / 64];
  int plan[4];
  float p[4][16][8];                           // per wave: p[token][head]
  float m[4][8], l[4][8];
  float acc[4][8][D];
};

template <int D, int G, bool LOCAL>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, DecodeShared<D, G>& sh, int item,
                                            int bg, int split, int chunk) {
  using TL = Tile<D>;
  constexpr int KS = TL::KS, NCLS = TL::NCLS, VT = TL::VT;
  constexpr int DPL = D / 4;                   // K elements per lane
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
  const int start = split * chunk;
  const int len = min(chunk, count - start);
  const int64_t row0 = (int64_t)bg * a.n_cap;

  // query fragment: head (lane % 16), this lane's slice of the k mapping
  bf16x8 qf[KS];
  {
    const int h = lane & 15, jq = lane >> 4;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (h < G) {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                             ((int64_t)b * a.Hq + g * G + h) * D + jq * DPL + 8 * s;
        w = *reinterpret_cast<const u32x4*>(qp);
      }
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // this wave's contiguous share of the item, in whole 16-token tiles
  const int per_wave = (((len + 3) / 4) + 15) & ~15;
  const int w0 = start + wid * per_wave, w1 = min(start + len, w0 + per_wave);
  const int ntiles = (w1 > w0) ? (w1 - w0 + 15) / 16 : 0;

  const int kt = lane & 15, jg = lane >> 4;            // K role
  const int vd = 2 * (lane % (D / 2)), vc = lane / (D / 2);   // V role
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + row0 * D + jg * DPL;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + row0 * D + vd;

  // raw list entry of this lane's token in a tile (a load for listed groups,
  // in bounds even past the end; checked when it is used)
  auto raw_id = [&](int tile) __attribute__((always_inline)) -> int {
    const int e = w0 + tile * 16 + kt;
    if (LOCAL) return (e < s_eff) ? e : wst + (e - s_eff);
    return a.sel_idx[row0 + min(e, w1 - 1)];
  };
  // issue a tile's K and V loads
  auto issue = [&](int tile, TL& t, int raw) __attribute__((always_inline)) {
    const int e = w0 + tile * 16 + kt;
    const int tok = (e < w1 && (unsigned)raw < (unsigned)n) ? raw : -1;
    t.tok = tok;
    const uint16_t* kp = kbase + (int64_t)max(tok, 0) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) t.k[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kp + 8 * s));
#pragma unroll
    for (int r = 0; r < VT; ++r) {
      int tv = __builtin_amdgcn_readlane(tok, r * NCLS);
      if (NCLS == 2) {
        const int tv1 = __builtin_amdgcn_readlane(tok, r * NCLS + 1);
        tv = vc ? tv1 : tv;
      }
      t.v[r] = *reinterpret_cast<const uint32_t*>(vbase + (int64_t)max(tv, 0) * D);
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
    for (int i = 0; i < 4; ++i) sv[i] = valid ? c[i] * sc : -INFINITY;
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

template <int D, int G>
__global__ __launch_bounds__(kMfmaThreads, (G > 4 ? 1 : 2)) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ DecodeShared<D, G> sh;
  const int chunk = plan_chunk(a, sh.scan64);
  plan_walk(a, chunk, blockIdx.x, -1, sh.scan32, sh.plan);
  const int bg = sh.plan[0], split = sh.plan[1];
  if (bg < 0) return;
  if ((a.local_mask >> (bg % a.Hkv)) & 1ull) decode_item<D, G, true>(a, sh, blockIdx.x, bg, split, chunk);
  else decode_item<D, G, false>(a, sh, blockIdx.x, bg, split, chunk);
}

// Merge the items of one (sequence, query head): weights 2^(m_i - M) per
// item, then every thread sums one output dim over its share of the items.
template <int D>
__global__ __launch_bounds__(kMfmaThreads) void decode_item_combine_kernel(DecodeArgs a) {
  constexpr int P = kMfmaThreads / D;          // item shares per output dim
  __shared__ int64_t s_scan64[kMfmaThreads / 64];
  __shared__ int s_scan32[kMfmaThreads / 64];
  __shared__ int s_plan[4];
  __shared__ float s_w[kMaxItemsLds];
  __shared__ float s_red[kMfmaThreads];
  __shared__ float s_M, s_L;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq, g = h / a.G, hh = h % a.G;
  const int chunk = plan_chunk(a, s_scan64);
  plan_walk(a, chunk, -1, b * a.Hkv + g, s_scan32, s_plan);
  const int first = s_plan[2], ns = min(s_plan[3], kMaxItemsLds);
  const int64_t stride = (int64_t)a.G * (D + 2);
  const float* base = a.partial + ((int64_t)first * a.G + hh) * (D + 2);
  float mx = -INFINITY;
  for (int sp = tid; sp < ns; sp += kMfmaThreads) mx = fmaxf(mx, base[sp * stride + D]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) s_red[tid >> 6] = mx;
  __syncthreads();
  if (tid == 0) s_M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  const float M = s_M;
  float lsum = 0.f;
  for (int sp = tid; sp < ns; sp += kMfmaThreads) {
    const float* q = base + sp * stride;
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
  for (int sp = part; sp < ns; sp += P) acc = fmaf(s_w[sp], base[sp * stride + e], acc);
  s_red[tid] = acc;
  __syncthreads();
  if (part == 0) {
    float v = acc;
#pragma unroll
    for (int q = 1; q < P; ++q) v += s_red[q * D + e];
    const float L = s_L;
    a.out[(int64_t)bh * D + e] = (L > 0.f) ? v / L : 0.f;
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int d, hipStream_t s) {
  if (a.max_splits < 1 || a.max_splits > kMaxItemsLds || a.target_items < 1) return hipErrorInvalidValue;
  dim3 grid(a.max_splits), block(kMfmaThreads);
#define SA_DEC(D_, G_) hipLaunchKernelGGL((decode_mfma_kernel<D_, G_>), grid, block, 0, s, a)
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
  if (d == 128) hipLaunchKernelGGL((decode_item_combine_kernel<128>), dim3(a.B * a.Hq), block, 0, s, a);
  else hipLaunchKernelGGL((decode_item_combine_kernel<64>), dim3(a.B * a.Hq), block, 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
