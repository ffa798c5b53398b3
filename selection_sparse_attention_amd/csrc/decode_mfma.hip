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
//   * the next tile's K and V loads are in flight while a tile is computed.
// Splits are merged by the same combine kernel as the fp32 path.
#include "args.hpp"
#include "common.hpp"

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

template <int D>
struct Tile {
  static constexpr int KS = D / 32;            // MFMA k-steps
  static constexpr int NCLS = 128 / D;         // token classes for the V pairs
  static constexpr int VT = 16 / NCLS;         // V rows per lane per tile
  bf16x8 k[KS];
  uint32_t v[VT];
};

template <int D, int G>
__global__ __launch_bounds__(kMfmaThreads) void decode_mfma_kernel(DecodeArgs a) {
  using TL = Tile<D>;
  constexpr int KS = TL::KS, NCLS = TL::NCLS, VT = TL::VT;
  constexpr int DPL = D / 4;                   // K elements per lane
  constexpr int HG = (G + 3) / 4;              // lane groups holding heads
  static_assert(G <= 8, "at most 8 query heads per KV group");
  __shared__ int s_list[kMaxTps + 64];
  __shared__ float s_p[4][16][8];              // per wave: p[token][head]
  __shared__ float s_m[4][8], s_l[4][8];
  __shared__ float s_acc[4][8][D];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
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
  const int64_t row0 = ((int64_t)b * a.Hkv + g) * a.n_cap;

  // this split's token positions, staged once
  for (int i = tid; i < end - start; i += kMfmaThreads) {
    const int e = start + i;
    int tok = local ? (e < s_eff ? e : ws + (e - s_eff)) : a.sel_idx[row0 + e];
    s_list[i] = ((unsigned)tok < (unsigned)n) ? tok : -1;
  }
  // query fragment: head (lane % 16), this lane's slice of the k mapping
  bf16x8 qf[KS];
  {
    const int h = lane & 15, jg = lane >> 4;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (h < G) {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                             ((int64_t)b * a.Hq + g * G + h) * D + jg * DPL + 8 * s;
        uint4 w = *reinterpret_cast<const uint4*>(qp);
        qf[s] = __builtin_bit_cast(bf16x8, w);
      } else {
        qf[s] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
      }
    }
  }
  __syncthreads();

  // this wave's contiguous share of the split
  const int len = end - start;
  const int per_wave = (((len + 3) / 4) + 15) & ~15;   // whole 16-token tiles
  const int w0 = wid * per_wave, w1 = min(len, w0 + per_wave);
  const int ntiles = (w1 > w0) ? (w1 - w0 + 15) / 16 : 0;

  const int kt = lane & 15, jg = lane >> 4;            // K role
  const int vd = 2 * (lane % (D / 2)), vc = lane / (D / 2);   // V role
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k);
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v);

  auto load_tile = [&](TL& t, int tile) {
    const int i0 = w0 + tile * 16;
    const int ik = i0 + kt;
    const int tok = (ik < w1) ? s_list[ik] : -1;
    if (tok >= 0) {
      const uint16_t* kp = kbase + (row0 + tok) * D + jg * DPL;
#pragma unroll
      for (int s = 0; s < KS; ++s)
        t.k[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kp + 8 * s));
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) t.k[s] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
    // the tile's 16 positions, read as a broadcast (i0 is a multiple of 16)
    int idx16[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int4 w = *reinterpret_cast<const int4*>(&s_list[i0 + 4 * q4]);
      idx16[4 * q4 + 0] = w.x; idx16[4 * q4 + 1] = w.y;
      idx16[4 * q4 + 2] = w.z; idx16[4 * q4 + 3] = w.w;
    }
#pragma unroll
    for (int r = 0; r < VT; ++r) {
      const int iv = i0 + r * NCLS + vc;
      const int tv0 = idx16[r * NCLS], tv1 = idx16[r * NCLS + (NCLS - 1)];
      const int tv = (iv < w1) ? (vc ? tv1 : tv0) : -1;
      t.v[r] = (tv >= 0) ? *reinterpret_cast<const uint32_t*>(vbase + (row0 + tv) * D + vd) : 0u;
    }
  };

  float m[G], lsum[4], acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; acc[h][0] = 0.f; acc[h][1] = 0.f; }
#pragma unroll
  for (int i = 0; i < 4; ++i) lsum[i] = 0.f;
  const float sc = a.scale_log2;

  auto compute_tile = [&](const TL& t, int tile) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[s], t.k[s], c, 0, 0, 0);
    const int i0 = w0 + tile * 16;
    const bool valid = (i0 + kt < w1) && (s_list[i0 + kt] >= 0);
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = valid ? c[i] * sc : -INFINITY;
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int grp = h >> 2, r = h & 3;
      const float tm = row16_max(sv[r]);
      const float tmax =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tm), 16 * grp));
      const float mn = fmaxf(m[h], tmax);
      alpha[h] = (m[h] == mn) ? 1.f : exp2f(m[h] - mn);
      m[h] = mn;
      if (jg == grp) {
        const float p = (sv[r] == -INFINITY) ? 0.f : exp2f(sv[r] - mn);
        lsum[r] = lsum[r] * alpha[h] + p;
        s_p[wid][kt][h] = p;
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int h = 0; h < G; ++h) { acc[h][0] *= alpha[h]; acc[h][1] *= alpha[h]; }
#pragma unroll
    for (int r = 0; r < VT; ++r) {
      const int tt = r * NCLS + vc;
      const float v0 = bf16_lo(t.v[r]), v1 = bf16_hi(t.v[r]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = s_p[wid][tt][h];
        acc[h][0] = fmaf(p, v0, acc[h][0]);
        acc[h][1] = fmaf(p, v1, acc[h][1]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  TL ta, tb;
  if (ntiles > 0) load_tile(ta, 0);
  for (int tile = 0; tile < ntiles; tile += 2) {
    if (tile + 1 < ntiles) load_tile(tb, tile + 1);
    compute_tile(ta, tile);
    if (tile + 1 < ntiles) {
      if (tile + 2 < ntiles) load_tile(ta, tile + 2);
      compute_tile(tb, tile + 1);
    }
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
  (void)HG;
  if (lane < D / 2) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_acc[wid][h][vd] = acc[h][0];
      s_acc[wid][h][vd + 1] = acc[h][1];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) { s_m[wid][h] = m[h]; s_l[wid][h] = (ntiles > 0) ? lw[h] : 0.f; }
    if (ntiles == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) s_m[wid][h] = -INFINITY;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kMfmaThreads) {
    const int h = idx / D, e = idx % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][h]);
    float av = 0.f, lv = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_m[w][h];
      const float wt = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      av += wt * s_acc[w][h][e];
      lv += wt * s_l[w][h];
    }
    float* pp = a.partial + (((int64_t)b * a.Hq + g * G + h) * a.max_splits + split) * (D + 2);
    pp[e] = av;
    if (e == 0) { pp[D] = M; pp[D + 1] = lv; }
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int d, hipStream_t s) {
  dim3 grid(a.max_splits, a.Hkv, a.B), block(kMfmaThreads);
  if (a.tps > kMaxTps) return hipErrorInvalidValue;
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
  return hipGetLastError();
}

}  // namespace sa
