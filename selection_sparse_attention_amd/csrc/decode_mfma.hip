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
// that group's item count; with `table`, also writes (first item, item
// count) of every group there.
__device__ void plan_walk(const DecodeArgs& a, int chunk, int item, int want, int* s_scan,
                          int* s_out, int2* table) {
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
      if (table) table[bg] = make_int2(first, ns);
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
                             ((int64_t)b * a.Hq + g * G + h) * D + 32 * s + 8 * jq;
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
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + row0 * D + 8 * jg;
  // V rows: a wave-uniform row address (scalar) plus this lane's dims
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + row0 * D;

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
  // workgroup 0 also records every group's items for the combine launch
  plan_walk(a, chunk, blockIdx.x, -1, sh.scan32, sh.plan, blockIdx.x == 0 ? a.plan : nullptr);
  const int bg = sh.plan[0], split = sh.plan[1];
  if (bg < 0) return;
  if ((a.local_mask >> (bg % a.Hkv)) & 1ull) decode_item<D, G, true>(a, sh, blockIdx.x, bg, split, chunk);
  else decode_item<D, G, false>(a, sh, blockIdx.x, bg, split, chunk);
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
    a.out[((int64_t)b * a.Hq + g * G + h) * D + e] = (L > 0.f) ? v / L : 0.f;
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int d, hipStream_t s) {
  if (a.max_splits < 1 || a.target_items < 1 || !a.plan) return hipErrorInvalidValue;
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

}  // namespace sa
