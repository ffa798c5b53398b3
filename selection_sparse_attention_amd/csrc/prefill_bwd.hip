// Backward pass of the pyramid-selection prefill (Lighthouse summary,
// Methodology 2B: the top-K choice is discrete and gets no gradient, which
// flows only through the gather, the attention on the gathered subsequence
// and the scatter back; 2A: a level-l entry is the mean of the p^l level-0
// rows it covers, so its gradient reaches each of them divided by p^l).
//
// Per query block beta and head, with the forward's key sequence (the
// block's chosen entries, then its own level-0 keys up to each query),
// a = q.k / sqrt(d), P = softmax(a) (recomputed from the stored log-sum-exp)
// and dO the upstream gradient:
//   dV_j += sum_i P_ij dO_i,  dA_ij = P_ij (dO_i.v_j - delta_i),  delta_i = dO_i.O_i,
//   dQ_i  = sum_j dA_ij k_j / sqrt(d),  dK_j += sum_i dA_ij q_i / sqrt(d).
//
// Stages (one stream, every sum in a fixed order: the result is the same
// from run to run):
//   1. init: delta per query; every entry's `last` block set to -1.
//   2. interval: per (head, block), the block's list and its two
//      neighbours' lists sorted in LDS; a chosen entry that the next block
//      drops records this block as its last.  The pyramid selection keeps an
//      entry from the first block that sees it through a last block (the
//      visible set only grows, so an entry's rank only falls); a list that
//      breaks this shape, repeats an id or holds one outside the pyramid
//      flags its head, whose gradients then come out NaN.
//   3. prefix: per head, an exclusive scan over the flat ids numbers each
//      entry's partial rows - one per choosing block, in block order, after
//      one for a level-0 key's own block.
//   4. dQ: per (block, head), the forward's walk over 32-key tiles gathered
//      into LDS (K, V row-major for S^T = K Q^T and dP^T = V dO^T with the
//      wave's queries resident, K^T for dQ^T += K^T dS^T).
//   5. dK/dV: per (block, head), the block's Q and dO staged once in LDS,
//      row-major and transposed; each wave takes 16 keys of the sequence at
//      a time with their K and V rows as matrix-core operands straight from
//      memory, forms S and dP over all 128 queries, and writes the block's
//      contribution to each key as one bf16 partial row (dV = dO^T P,
//      dK = Q^T dS).
//   6. reduce: each entry's partial rows summed in fp32 in block order;
//      coarse entries first, then each level-0 row adds its ancestors'
//      sums / p^l.
//
// Matrix-core products are v_mfma_f32_16x16x32_bf16 with fp32 accumulation;
// P, dS and dO enter them rounded once to bf16, as do the partial rows.
#include <algorithm>

#include "args.hpp"
#include "common.hpp"

namespace sa {
namespace {

typedef __bf16 bf16x8b __attribute__((ext_vector_type(8)));
typedef float f32x4b __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4b __attribute__((ext_vector_type(4)));
typedef float f32x2b __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2b __attribute__((ext_vector_type(2)));

constexpr int kD = 128;                 // head dim
constexpr int kRowB = kD * 2;           // bytes of one bf16 row
constexpr int kListMaxB = 8192;         // longest list (block_top_k)
constexpr uint32_t kCoarseB = 0x80000000u;
constexpr float kLog2e = 1.4426950408889634f;

// fp32 pair -> packed bf16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2b){x, y}, bf16x2b));
}

// The per-level tables are read with constant indices only: a lane-dependent
// index into the argument block would become a vector load, and its wait
// would also wait for every store the wave still has in flight.

// one past the last position that flat entry f covers
__device__ __forceinline__ int64_t span_end(const BwdArgs& a, int32_t f) {
  int o = a.off[0], sp = a.span[0];
#pragma unroll
  for (int m = 1; m < 8; ++m)
    if (m < a.levels && f >= a.off[m]) { o = a.off[m]; sp = a.span[m]; }
  return (int64_t)(f - o + 1) * sp;
}

// first block that sees flat entry f: its span must end at or before the
// block's first query
__device__ __forceinline__ int first_block(const BwdArgs& a, int32_t f) {
  return (int)((span_end(a, f) + a.q_block - 1) / a.q_block);
}

// byte offset of flat entry f's K/V row (level 0 in k/v, coarse in pk/pv
// with the top bit set); ids outside the pyramid read level-0 row 0
__device__ __forceinline__ uint32_t row_of(const BwdArgs& a, int32_t f) {
  if ((unsigned)f < (unsigned)a.N) return (uint32_t)f * kRowB;
  if ((unsigned)(f - a.N) < (unsigned)a.Nc) return (uint32_t)(f - a.N) * kRowB | kCoarseB;
  return 0u;
}

// (head, block) of workgroup L: heavy blocks first, two heads per die
__device__ __forceinline__ bool unit_of(const BwdArgs& a, int L, int& bh, int& blk) {
  const int nh = a.B * a.H;
  const int hpx = (nh + 7) / 8;
  const int xcd = L % 8, slot = L / 8;
  bh = xcd + 8 * (slot % hpx);
  blk = a.nblk - 1 - slot / hpx;
  return bh < nh && blk >= 0;
}

}  // namespace

// ---------------------------------------------------------------- 1. init
__global__ __launch_bounds__(256) void bwd_init_kernel(BwdArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nthreads = (int64_t)gridDim.x * 256;
  const int64_t n_last = (int64_t)a.B * a.H * a.E;
  for (int64_t i = gid; i < n_last; i += nthreads) a.last[i] = -1;
  if (gid < (int64_t)a.B * a.H) a.err[gid] = 0u;
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  for (int64_t row = gid >> 6; row < rows; row += nthreads >> 6) {
    const float2 o = reinterpret_cast<const float2*>(a.out + row * kD)[lane];
    const float2 g = reinterpret_cast<const float2*>(a.dout + row * kD)[lane];
    float s = o.x * g.x + o.y * g.y;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (lane == 0) a.delta[row] = s;
  }
}

// ---------------------------------------------------------------- 2. interval
constexpr int kIvThreads = 256;

__device__ __forceinline__ bool in_sorted(const int32_t* x, int n, int32_t v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (x[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo < n && x[lo] == v;
}

// Dynamic LDS: the lists of blocks blk - 1, blk and blk + 1, P ids each (P a
// power of two >= block_top_k).  The pyramid selection writes its lists in
// ascending order; lists in another order are sorted here first.
__global__ __launch_bounds__(kIvThreads) void bwd_interval_kernel(BwdArgs a, int P) {
  extern __shared__ int32_t s_dyn[];
  int32_t* s_l[3] = {s_dyn, s_dyn + P, s_dyn + 2 * P};
  const int blk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int32_t* cnts = a.blk_count + (int64_t)bh * a.nblk;
  int n[3];
  bool bad = false;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int b = blk - 1 + r;
    int c = 0;
    if (b >= 0 && b < a.nblk) {
      const int raw = cnts[b];
      if (raw < 0 && r == 1) bad = true;
      c = min(max(raw, 0), a.K);
    }
    n[r] = c;
  }
  int unsorted = 0;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const int32_t* lst = a.blk_idx + ((int64_t)bh * a.nblk + (blk - 1 + r)) * a.K;
    for (int i = tid; i < P; i += kIvThreads) {
      const int32_t v = (i < n[r]) ? lst[i] : INT32_MAX;
      s_l[r][i] = v;
      if (i + 1 < n[r] && v >= lst[i + 1]) unsorted = 1;
    }
  }
  if (__syncthreads_or(unsorted)) {
    // ascending bitonic sort of the three lists together
    for (int k = 2; k <= P; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P; i += kIvThreads) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const bool up = (i & k) == 0;
#pragma unroll
            for (int r = 0; r < 3; ++r) {
              const int32_t u = s_l[r][i], w = s_l[r][ixj];
              if ((u > w) == up) { s_l[r][i] = w; s_l[r][ixj] = u; }
            }
          }
        }
        __syncthreads();
      }
    }
  }
  int32_t* last = a.last + (int64_t)bh * a.E;
  for (int s = tid; s < n[1]; s += kIvThreads) {
    const int32_t f = s_l[1][s];
    bool ok = f >= 0 && f < a.E && (s == 0 || s_l[1][s - 1] != f);
    if (ok) {
      const int64_t end = span_end(a, f);
      const int b0 = (int)((end + a.q_block - 1) / a.q_block);
      ok = end <= (int64_t)a.q_block * blk;               // visible to this block
      if (ok && blk > b0) ok = in_sorted(s_l[0], n[0], f); // chosen without a gap since b0
      if (ok && (blk == a.nblk - 1 || !in_sorted(s_l[2], n[2], f))) last[f] = blk;
    }
    if (!ok) bad = true;
  }
  if (__syncthreads_or(bad) && tid == 0) atomicOr(a.err + bh, 1u);
}

// ---------------------------------------------------------------- 3. prefix
constexpr int kPxThreads = 1024;

__global__ __launch_bounds__(kPxThreads) void bwd_prefix_kernel(BwdArgs a) {
  __shared__ int32_t s_scan[kPxThreads / 64];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int E = a.E;
  const int per = (E + kPxThreads - 1) / kPxThreads;
  const int lo = min(E, tid * per), hi = min(E, lo + per);
  const int32_t* last = a.last + (int64_t)bh * E;
  auto len_of = [&](int f) -> int32_t {
    const int32_t l = last[f];
    int32_t c = (f < a.N) ? 1 : 0;
    if (l >= 0) c += l - first_block(a, f) + 1;
    return c;
  };
  int32_t sum = 0;
  for (int f = lo; f < hi; ++f) sum += len_of(f);
  int32_t total;
  int32_t run = block_exclusive_scan<int32_t, kPxThreads>(sum, s_scan, &total);
  int32_t* base = a.base + (int64_t)bh * (E + 1);
  for (int f = lo; f < hi; ++f) {
    base[f] = run;
    run += len_of(f);
  }
  if (tid == 0) base[E] = total;
}

// ---------------------------------------------------------------- 4. dQ
constexpr int kDqThreads = 256;
constexpr int kKT = 32;                 // keys per tile
constexpr int kKRow = kD + 8;           // row-major tile stride (bf16 elements)
constexpr int kTRow = 36;               // transposed tile stride (bf16 elements)

__global__ __launch_bounds__(kDqThreads, 2) void bwd_dq_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kKT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[2][kKT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t s_kt[2][kD * kTRow];
  int bh, blk;
  if (!unit_of(a, blockIdx.x, bh, blk)) return;
  if (a.err[bh]) return;                          // the reduce writes NaN for this head
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, jg = lane >> 4;
  const int q0 = blk * a.q_block;
  const int nq = min(a.q_block, a.N - q0);
  const int c_sel = min(max(a.blk_count[(int64_t)bh * a.nblk + blk], 0), a.K);
  const int32_t* list = a.blk_idx + ((int64_t)bh * a.nblk + blk) * a.K;
  const int T = c_sel + nq;
  const int ntiles = (T + kKT - 1) / kKT;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)bh * a.N * kD;
  const float* dob = a.dout + (int64_t)bh * a.N * kD;
  const char* kb = reinterpret_cast<const char*>(a.k) + (int64_t)bh * a.N * kRowB;
  const char* vb = reinterpret_cast<const char*>(a.v) + (int64_t)bh * a.N * kRowB;
  const char* pkb = a.Nc ? reinterpret_cast<const char*>(a.pk) + (int64_t)bh * a.Nc * kRowB : kb;
  const char* pvb = a.Nc ? reinterpret_cast<const char*>(a.pv) + (int64_t)bh * a.Nc * kRowB : vb;

  // resident B operands: queries 32w + 16nt + l16, dims 32jg + 8s .. +8
  bf16x8b qf[2][4], df[2][4];
  float lq[2], dl[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int ql = 32 * wid + 16 * nt + l16;
    const bool valid = ql < nq;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 w = make_uint4(0, 0, 0, 0);
      float4 g0 = make_float4(0.f, 0.f, 0.f, 0.f), g1 = g0;
      if (valid) {
        w = *reinterpret_cast<const uint4*>(qb + (int64_t)(q0 + ql) * kD + 32 * jg + 8 * s);
        const float4* gp = reinterpret_cast<const float4*>(dob + (int64_t)(q0 + ql) * kD + 32 * jg + 8 * s);
        g0 = gp[0];
        g1 = gp[1];
      }
      qf[nt][s] = __builtin_bit_cast(bf16x8b, w);
      df[nt][s] = __builtin_bit_cast(bf16x8b, make_uint4(pack_bf16(g0.x, g0.y), pack_bf16(g0.z, g0.w),
                                                         pack_bf16(g1.x, g1.y), pack_bf16(g1.z, g1.w)));
    }
    lq[nt] = valid ? a.lse[(int64_t)bh * a.N + q0 + ql] * kLog2e : INFINITY;
    dl[nt] = valid ? a.delta[(int64_t)bh * a.N + q0 + ql] : 0.f;
  }

  // key sequence entry e with list entry f -> row byte offset (past the
  // end: row 0, masked)
  auto seq_row = [&](int e, int32_t f) __attribute__((always_inline)) -> uint32_t {
    if (e < c_sel) return row_of(a, f);
    if (e < T) return (uint32_t)(q0 + e - c_sel) * kRowB;
    return 0u;
  };
  auto list_at = [&](int e) __attribute__((always_inline)) -> int32_t {
    return (e < c_sel) ? list[e] : 0;
  };
  auto rptr = [](uint32_t r, const char* b0, const char* bc) __attribute__((always_inline)) {
    return reinterpret_cast<const u32x4b*>((((int32_t)r < 0) ? bc : b0) + (r & ~kCoarseB));
  };
  // gather roles: row-major tiles (key tid/8, 16 B at 16 (tid%8) and 128 B
  // further) and the transposed K tile (keys 2 (tid%16) and +1, dims 8 (tid/16) .. +8)
  const int gk_key = tid >> 3, gk_seg = tid & 7;
  const int gt_kp = tid & 15, gt_seg = tid >> 4;
  struct Rows { u32x4b k0, k1, v0, v1, t0, t1; };
  // the list entries of this thread's three rows of tile x
  struct Ids { int32_t a, b0, b1; };
  auto ids_of = [&](int x) __attribute__((always_inline)) -> Ids {
    return Ids{list_at(x * kKT + gk_key), list_at(x * kKT + 2 * gt_kp), list_at(x * kKT + 2 * gt_kp + 1)};
  };
  auto gather = [&](int x, const Ids& id, Rows& r) __attribute__((always_inline)) {
    const uint32_t ra = seq_row(x * kKT + gk_key, id.a);
    const u32x4b* pk = rptr(ra, kb + 16 * gk_seg, pkb + 16 * gk_seg);
    const u32x4b* pv = rptr(ra, vb + 16 * gk_seg, pvb + 16 * gk_seg);
    r.k0 = pk[0];
    r.k1 = pk[8];
    r.v0 = pv[0];
    r.v1 = pv[8];
    const uint32_t rb0 = seq_row(x * kKT + 2 * gt_kp, id.b0), rb1 = seq_row(x * kKT + 2 * gt_kp + 1, id.b1);
    r.t0 = *rptr(rb0, kb + 16 * gt_seg, pkb + 16 * gt_seg);
    r.t1 = *rptr(rb1, kb + 16 * gt_seg, pkb + 16 * gt_seg);
  };
  auto stash = [&](int buf, const Rows& r) __attribute__((always_inline)) {
    uint16_t* kd = s_k[buf] + gk_key * kKRow + 8 * gk_seg;
    *reinterpret_cast<u32x4b*>(kd) = r.k0;
    *reinterpret_cast<u32x4b*>(kd + 64) = r.k1;
    uint16_t* vd = s_v[buf] + gk_key * kKRow + 8 * gk_seg;
    *reinterpret_cast<u32x4b*>(vd) = r.v0;
    *reinterpret_cast<u32x4b*>(vd + 64) = r.v1;
    // K^T: dims 8 gt_seg + i, keys 2 gt_kp and 2 gt_kp + 1 packed in one dword
    uint16_t* td = s_kt[buf] + (8 * gt_seg) * kTRow + 2 * gt_kp;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint32_t*>(td + (2 * i) * kTRow) = __builtin_amdgcn_perm(r.t1[i], r.t0[i], 0x05040100u);
      *reinterpret_cast<uint32_t*>(td + (2 * i + 1) * kTRow) = __builtin_amdgcn_perm(r.t1[i], r.t0[i], 0x07060302u);
    }
  };
  // S^T-shaped product of a row-major tile with resident fragments:
  // out[mt][nt] = rows 16 mt + 4 jg + i, queries 16 nt + l16
  auto rows_x_frags = [&](const uint16_t* tile, const bf16x8b (&fr)[2][4], f32x4b (&out)[2][2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      bf16x8b af[4];
#pragma unroll
      for (int st = 0; st < 4; ++st)
        af[st] = __builtin_bit_cast(bf16x8b, *reinterpret_cast<const uint4*>(tile + (16 * mt + l16) * kKRow + 32 * jg + 8 * st));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4b c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[st], fr[nt][st], c, 0, 0, 0);
        out[mt][nt] = c;
      }
    }
  };

  f32x4b acc[8][2];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[dt][nt] = (f32x4b){0.f, 0.f, 0.f, 0.f};
  const float sc = a.scale_log2;

  Rows cur;
  gather(0, ids_of(0), cur);
  stash(0, cur);
  Ids id_next = ids_of(1);
  // nothing in flight on entry: loads pending into registers that the loop
  // reuses would otherwise put a full wait before every tile's first product
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    Rows nxt;
    const bool more = t + 1 < ntiles;
    Ids id_after{0, 0, 0};
    if (more) {
      gather(t + 1, id_next, nxt);
      id_after = ids_of(t + 2);
    }
    f32x4b s[2][2], dp[2][2];
    rows_x_frags(s_k[buf], qf, s);
    rows_x_frags(s_v[buf], df, dp);
    // dS^T, packed as the B operand of dQ^T += K^T dS^T: k-slot 8 jg + j is
    // key 4 jg + j (j < 4) or 16 + 4 jg + (j - 4)
    uint4 dsp[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int ql = 32 * wid + 16 * nt + l16;
      float ds[8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = t * kKT + 16 * mt + 4 * jg + i;
          const bool ok = (e < c_sel) || (e < T && (e - c_sel) <= ql);
          const float p = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][nt][i], sc, -lq[nt])) : 0.f;
          ds[4 * mt + i] = p * (dp[mt][nt][i] - dl[nt]);
        }
      dsp[nt] = make_uint4(pack_bf16(ds[0], ds[1]), pack_bf16(ds[2], ds[3]),
                           pack_bf16(ds[4], ds[5]), pack_bf16(ds[6], ds[7]));
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* trow = s_kt[buf] + (16 * dt + l16) * kTRow;
      const uint2 w0 = *reinterpret_cast<const uint2*>(trow + 4 * jg);
      const uint2 w1 = *reinterpret_cast<const uint2*>(trow + 16 + 4 * jg);
      const bf16x8b kt = __builtin_bit_cast(bf16x8b, make_uint4(w0.x, w0.y, w1.x, w1.y));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, __builtin_bit_cast(bf16x8b, dsp[nt]), acc[dt][nt], 0, 0, 0);
    }
    if (more) stash(buf ^ 1, nxt);
    id_next = id_after;
    __syncthreads();
  }

  // lane holds d = 16 dt + 4 jg + 0..3 of query 32 w + 16 nt + l16
  float* dqb = a.dq + (int64_t)bh * a.N * kD;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int ql = 32 * wid + 16 * nt + l16;
    if (ql < nq) {
      float* row = dqb + (int64_t)(q0 + ql) * kD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4b v = acc[dt][nt] * a.scale;
        *reinterpret_cast<float4*>(row + 16 * dt + 4 * jg) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// ---------------------------------------------------------------- 5. dK / dV partials
constexpr int kKvThreads = 512;
constexpr int kQRow = kD + 8;           // row-major staged tile stride (bf16 elements)
constexpr int kQtRow = kD + 4;          // transposed staged tile stride: 66 dwords, so the
                                        // 8-byte reads of 16 lanes (16 rows) hit distinct banks

__global__ __launch_bounds__(kKvThreads, 1) void bwd_dkv_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_q[128 * kQRow];    // Q[q][d]
  __shared__ __attribute__((aligned(16))) uint16_t s_qt[128 * kQtRow];  // Q^T[d][q]
  __shared__ __attribute__((aligned(16))) uint16_t s_do[128 * kQRow];   // dO[q][d]
  __shared__ __attribute__((aligned(16))) uint16_t s_dot[128 * kQtRow]; // dO^T[d][q]
  __shared__ __attribute__((aligned(16))) float s_lse[128];
  __shared__ __attribute__((aligned(16))) float s_dl[128];
  int bh, blk;
  if (!unit_of(a, blockIdx.x, bh, blk)) return;
  if (a.err[bh]) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, jg = lane >> 4;
  const int q0 = blk * a.q_block;
  const int nq = min(a.q_block, a.N - q0);
  const int c_sel = min(max(a.blk_count[(int64_t)bh * a.nblk + blk], 0), a.K);
  const int32_t* list = a.blk_idx + ((int64_t)bh * a.nblk + blk) * a.K;
  const int T = c_sel + nq;
  const char* kb = reinterpret_cast<const char*>(a.k) + (int64_t)bh * a.N * kRowB;
  const char* vb = reinterpret_cast<const char*>(a.v) + (int64_t)bh * a.N * kRowB;
  const char* pkb = a.Nc ? reinterpret_cast<const char*>(a.pk) + (int64_t)bh * a.Nc * kRowB : kb;
  const char* pvb = a.Nc ? reinterpret_cast<const char*>(a.pv) + (int64_t)bh * a.Nc * kRowB : vb;

  // ---- stage the block's Q and dO (bf16), row-major and transposed; rows
  //      past the block's end are zero and their lse is +inf (P = 0)
  {
    const int row = tid >> 2, c0 = 32 * (tid & 3);
    const bool valid = row < nq;
    const uint16_t* qr = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)bh * a.N + q0 + row) * kD + c0;
    const float* gr = a.dout + ((int64_t)bh * a.N + q0 + row) * kD + c0;
    uint32_t qw[16], gw[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint4 w = make_uint4(0, 0, 0, 0);
      float4 g0 = make_float4(0.f, 0.f, 0.f, 0.f), g1 = g0;
      if (valid) {
        w = reinterpret_cast<const uint4*>(qr)[u];
        g0 = reinterpret_cast<const float4*>(gr)[2 * u];
        g1 = reinterpret_cast<const float4*>(gr)[2 * u + 1];
      }
      qw[4 * u] = w.x; qw[4 * u + 1] = w.y; qw[4 * u + 2] = w.z; qw[4 * u + 3] = w.w;
      gw[4 * u] = pack_bf16(g0.x, g0.y);
      gw[4 * u + 1] = pack_bf16(g0.z, g0.w);
      gw[4 * u + 2] = pack_bf16(g1.x, g1.y);
      gw[4 * u + 3] = pack_bf16(g1.z, g1.w);
      *reinterpret_cast<uint4*>(s_q + row * kQRow + c0 + 8 * u) =
          make_uint4(qw[4 * u], qw[4 * u + 1], qw[4 * u + 2], qw[4 * u + 3]);
      *reinterpret_cast<uint4*>(s_do + row * kQRow + c0 + 8 * u) =
          make_uint4(gw[4 * u], gw[4 * u + 1], gw[4 * u + 2], gw[4 * u + 3]);
    }
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      const int sh = (m & 1) * 16;
      s_qt[(c0 + m) * kQtRow + row] = (uint16_t)(qw[m >> 1] >> sh);
      s_dot[(c0 + m) * kQtRow + row] = (uint16_t)(gw[m >> 1] >> sh);
    }
    if (tid < 128) {
      const bool v = tid < nq;
      s_lse[tid] = v ? a.lse[(int64_t)bh * a.N + q0 + tid] * kLog2e : INFINITY;
      s_dl[tid] = v ? a.delta[(int64_t)bh * a.N + q0 + tid] : 0.f;
    }
  }
  __syncthreads();

  const float sc = a.scale_log2;
  const int32_t* base = a.base + (int64_t)bh * (a.E + 1);
  uint16_t* pkd = a.part_k + (int64_t)bh * a.R * kD;
  uint16_t* pvd = a.part_v + (int64_t)bh * a.R * kD;

  // Partial rows past the last real one go to the head's spare row, R - 1:
  // every lane stores every step, so the loop has no branch around its
  // stores and the waits for its prefetches count them exactly.
  const int64_t spare = a.R - 1;
  // the list entry of sequence entry e (read a step before its rows; the
  // read itself is always in bounds, K >= 1)
  auto list_at = [&](int e) __attribute__((always_inline)) -> int32_t {
    const int32_t v = list[min(e, a.K - 1)];
    return (e < c_sel) ? v : 0;
  };
  // this lane's key of a step: sequence entry e = step + 16 w + l16 with
  // list entry f -> row byte offset r, and the partial row as base[bi] + adj
  // (bi = -1: nothing to write); entries past the end read row 0
  auto key_of = [&](int e, int32_t f, uint32_t& r, int32_t& bi, int32_t& adj) __attribute__((always_inline)) {
    r = 0u;
    bi = -1;
    adj = 0;
    if (e < c_sel) {
      r = row_of(a, f);
      if ((unsigned)f < (unsigned)a.E) {
        bi = f;
        adj = (f < a.N ? 1 : 0) + (blk - first_block(a, f));
      }
    } else if (e < T) {
      const int32_t qf = q0 + e - c_sel;
      r = (uint32_t)qf * kRowB;
      bi = qf;
    }
  };
  auto part_row = [&](int32_t bi, int32_t bv, int32_t adj) __attribute__((always_inline)) -> int64_t {
    const int64_t pr = (int64_t)bv + adj;
    return (bi >= 0 && pr >= 0 && pr < spare) ? pr : spare;
  };
  auto load_frags = [&](uint32_t r, bf16x8b (&kf)[4], bf16x8b (&vf)[4]) __attribute__((always_inline)) {
    const bool coarse = (int32_t)r < 0;
    const char* kp = (coarse ? pkb : kb) + (r & ~kCoarseB) + 2 * (32 * jg);
    const char* vp = (coarse ? pvb : vb) + (r & ~kCoarseB) + 2 * (32 * jg);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      kf[st] = __builtin_bit_cast(bf16x8b, *reinterpret_cast<const uint4*>(kp + 16 * st));
      vf[st] = __builtin_bit_cast(bf16x8b, *reinterpret_cast<const uint4*>(vp + 16 * st));
    }
  };

  int e = 16 * wid + l16;
  uint32_t r;
  int64_t pr;
  {
    int32_t bi, adj;
    key_of(e, list_at(e), r, bi, adj);
    pr = part_row(bi, base[max(bi, 0)], adj);
  }
  bf16x8b kf[4], vf[4];
  load_frags(r, kf, vf);
  int32_t f_next = list_at(e + 128);
  // the first step's rows land before the loop: with loads still in flight
  // into kf/vf on entry, every step would wait for the next step's rows
  // before its first product
  __builtin_amdgcn_s_waitcnt(0);
  for (int step = 0; step < T; step += 128) {
    // the next step's key, base entry and rows, in flight under this step's
    // products, and the list entry of the step after it (issued also on the
    // last step, where they read in-bounds rows that nothing uses)
    const int en = e + 128;
    uint32_t rn;
    int32_t bin, adjn;
    bf16x8b kn[4], vn[4];
    key_of(en, f_next, rn, bin, adjn);
    const int32_t bvn = base[max(bin, 0)];
    load_frags(rn, kn, vn);
    const int32_t f_after = list_at(en + 128);
    // S[q][e] = Q K^T and dP[q][e] = dO V^T over all 128 queries, 32 at a
    // time (query group c: tiles qt = 2c, 2c + 1, rows q = 16 qt + 4 jg + i,
    // column e = l16).  Software-pipelined: group c + 1's products are issued
    // before group c's softmax work, so the two overlap within the wave.
    uint4 pb[4], db[4];
    const bool ev = e < T;
    auto products = [&](int c, f32x4b (&s2)[2], f32x4b (&d2)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qt = 2 * c + h;
        f32x4b cs = {0.f, 0.f, 0.f, 0.f}, cd = cs;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const bf16x8b aq = __builtin_bit_cast(bf16x8b, *reinterpret_cast<const uint4*>(s_q + (16 * qt + l16) * kQRow + 32 * jg + 8 * st));
          const bf16x8b ad = __builtin_bit_cast(bf16x8b, *reinterpret_cast<const uint4*>(s_do + (16 * qt + l16) * kQRow + 32 * jg + 8 * st));
          cs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, kf[st], cs, 0, 0, 0);
          cd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ad, vf[st], cd, 0, 0, 0);
        }
        s2[h] = cs;
        d2[h] = cd;
      }
    };
    // P and dS of group c, packed as B operands over queries 32 c .. 32 c + 31:
    // k-slot 8 jg + j is query 32 c + 4 jg + j (j < 4) or 32 c + 16 + 4 jg + (j - 4)
    auto softmax_grad = [&](int c, const f32x4b (&s2)[2], const f32x4b (&d2)[2]) __attribute__((always_inline)) {
      float p[8], ds[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 lv = *reinterpret_cast<const float4*>(s_lse + 32 * c + 16 * h + 4 * jg);
        const float4 dv = *reinterpret_cast<const float4*>(s_dl + 32 * c + 16 * h + 4 * jg);
        const float lvs[4] = {lv.x, lv.y, lv.z, lv.w};
        const float dvs[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ql = 32 * c + 16 * h + 4 * jg + i;
          const bool ok = ev && (e < c_sel || (e - c_sel) <= ql);
          const float pv = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(s2[h][i], sc, -lvs[i])) : 0.f;
          p[4 * h + i] = pv;
          ds[4 * h + i] = pv * (d2[h][i] - dvs[i]);
        }
      }
      pb[c] = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7]));
      db[c] = make_uint4(pack_bf16(ds[0], ds[1]), pack_bf16(ds[2], ds[3]), pack_bf16(ds[4], ds[5]), pack_bf16(ds[6], ds[7]));
    };
    {
      f32x4b sa[2], da[2], sb[2], db2[2];
      products(0, sa, da);
      __builtin_amdgcn_sched_barrier(0);
      products(1, sb, db2);
      softmax_grad(0, sa, da);
      __builtin_amdgcn_sched_barrier(0);
      products(2, sa, da);
      softmax_grad(1, sb, db2);
      __builtin_amdgcn_sched_barrier(0);
      products(3, sb, db2);
      softmax_grad(2, sa, da);
      __builtin_amdgcn_sched_barrier(0);
      softmax_grad(3, sb, db2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // dV^T[d][e] = sum_q dO^T[d][q] P[q][e], dK^T[d][e] = sum_q Q^T[d][q] dS[q][e]:
    // rows d = 16 dt + 4 jg + i, column e = l16; tile dt + 1's products are
    // issued before tile dt's results are packed and stored
    auto dvdk = [&](int dt, f32x4b& cv, f32x4b& ck) __attribute__((always_inline)) {
      cv = (f32x4b){0.f, 0.f, 0.f, 0.f};
      ck = cv;
      const uint16_t* vrow = s_dot + (16 * dt + l16) * kQtRow;
      const uint16_t* krow = s_qt + (16 * dt + l16) * kQtRow;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint2 v0 = *reinterpret_cast<const uint2*>(vrow + 32 * c + 4 * jg);
        const uint2 v1 = *reinterpret_cast<const uint2*>(vrow + 32 * c + 16 + 4 * jg);
        const uint2 k0 = *reinterpret_cast<const uint2*>(krow + 32 * c + 4 * jg);
        const uint2 k1 = *reinterpret_cast<const uint2*>(krow + 32 * c + 16 + 4 * jg);
        cv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8b, make_uint4(v0.x, v0.y, v1.x, v1.y)),
                                                     __builtin_bit_cast(bf16x8b, pb[c]), cv, 0, 0, 0);
        ck = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8b, make_uint4(k0.x, k0.y, k1.x, k1.y)),
                                                     __builtin_bit_cast(bf16x8b, db[c]), ck, 0, 0, 0);
      }
    };
    auto store = [&](int dt, f32x4b cv, f32x4b ck) __attribute__((always_inline)) {
      const int64_t o = pr * kD + 16 * dt + 4 * jg;
      *reinterpret_cast<uint2*>(pvd + o) = make_uint2(pack_bf16(cv[0], cv[1]), pack_bf16(cv[2], cv[3]));
      ck *= a.scale;
      *reinterpret_cast<uint2*>(pkd + o) = make_uint2(pack_bf16(ck[0], ck[1]), pack_bf16(ck[2], ck[3]));
    };
    {
      f32x4b va, ka, vb, kb2;
      dvdk(0, va, ka);
#pragma unroll
      for (int dt = 0; dt < 8; dt += 2) {
        __builtin_amdgcn_sched_barrier(0);
        dvdk(dt + 1, vb, kb2);
        store(dt, va, ka);
        __builtin_amdgcn_sched_barrier(0);
        if (dt + 2 < 8) dvdk(dt + 2, va, ka);
        store(dt + 1, vb, kb2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    e = en;
    r = rn;
    pr = part_row(bin, bvn, adjn);
    f_next = f_after;
#pragma unroll
    for (int st = 0; st < 4; ++st) { kf[st] = kn[st]; vf[st] = vn[st]; }
  }
}

// ---------------------------------------------------------------- 6. reduce
// Lane holds dims 2 lane, 2 lane + 1 of a row.  Sum of partial rows r0 + w,
// r0 + w + stride, ... < r1 of one entry (bf16 pairs, eight rows in flight).
__device__ __forceinline__ void sum_rows(const uint32_t* pk, const uint32_t* pv, int64_t r0,
                                         int64_t r1, int stride, float2& sk, float2& sv) {
  constexpr int U = 8;
  int64_t r = r0;
  for (; r + (int64_t)(U - 1) * stride < r1; r += (int64_t)U * stride) {
    uint32_t xk[U], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xk[u] = pk[(r + (int64_t)u * stride) * (kD / 2)];
      xv[u] = pv[(r + (int64_t)u * stride) * (kD / 2)];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      sk.x += __uint_as_float(xk[u] << 16);
      sk.y += __uint_as_float(xk[u] & 0xFFFF0000u);
      sv.x += __uint_as_float(xv[u] << 16);
      sv.y += __uint_as_float(xv[u] & 0xFFFF0000u);
    }
  }
  for (; r < r1; r += stride) {
    const uint32_t xk = pk[r * (kD / 2)], xv = pv[r * (kD / 2)];
    sk.x += __uint_as_float(xk << 16);
    sk.y += __uint_as_float(xk & 0xFFFF0000u);
    sv.x += __uint_as_float(xv << 16);
    sv.y += __uint_as_float(xv & 0xFFFF0000u);
  }
}

// Coarse entries (chosen by many blocks): one 256-thread workgroup per
// entry, wave w summing rows w, w + 4, ...; the four sums are added in wave
// order.
__global__ __launch_bounds__(256) void bwd_reduce_coarse_kernel(BwdArgs a) {
  __shared__ float2 s_k[4][64], s_v[4][64];
  const int bh = blockIdx.y, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int w = blockIdx.x;
  const int32_t f = a.N + w;
  const bool bad = a.err[bh] != 0;
  float2 sk = make_float2(0.f, 0.f), sv = sk;
  if (!bad) {
    const int32_t* base = a.base + (int64_t)bh * (a.E + 1);
    const uint32_t* pk = reinterpret_cast<const uint32_t*>(a.part_k) + (int64_t)bh * a.R * (kD / 2) + lane;
    const uint32_t* pv = reinterpret_cast<const uint32_t*>(a.part_v) + (int64_t)bh * a.R * (kD / 2) + lane;
    sum_rows(pk, pv, (int64_t)base[f] + wv, base[f + 1], 4, sk, sv);
  }
  s_k[wv][lane] = sk;
  s_v[wv][lane] = sv;
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int u = 1; u < 4; ++u) {
      sk.x += s_k[u][lane].x;
      sk.y += s_k[u][lane].y;
      sv.x += s_v[u][lane].x;
      sv.y += s_v[u][lane].y;
    }
    const int64_t o = ((int64_t)bh * a.Nc + w) * kD;
    reinterpret_cast<float2*>(a.coarse_k + o)[lane] = sk;
    reinterpret_cast<float2*>(a.coarse_v + o)[lane] = sv;
  }
}

// Level-0 rows: one wave per row, its own partial rows, then each coarse
// ancestor's sum divided by the rows it covers.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
  const int bh = blockIdx.y, lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.N) return;
  const bool bad = a.err[bh] != 0;
  float2 sk = make_float2(0.f, 0.f), sv = sk;
  if (!bad) {
    const int32_t* base = a.base + (int64_t)bh * (a.E + 1);
    const uint32_t* pk = reinterpret_cast<const uint32_t*>(a.part_k) + (int64_t)bh * a.R * (kD / 2) + lane;
    const uint32_t* pv = reinterpret_cast<const uint32_t*>(a.part_v) + (int64_t)bh * a.R * (kD / 2) + lane;
    sum_rows(pk, pv, base[w], base[w + 1], 1, sk, sv);
    for (int l = 1; l < a.levels; ++l) {
      const int j = w / a.span[l];
      if (j >= a.cnt[l]) continue;
      const int64_t o = ((int64_t)bh * a.Nc + (a.off[l] - a.N) + j) * kD;
      const float inv = 1.f / (float)a.span[l];
      const float2 ck = reinterpret_cast<const float2*>(a.coarse_k + o)[lane];
      const float2 cv = reinterpret_cast<const float2*>(a.coarse_v + o)[lane];
      sk.x += ck.x * inv;
      sk.y += ck.y * inv;
      sv.x += cv.x * inv;
      sv.y += cv.y * inv;
    }
  }
  const int64_t o = ((int64_t)bh * a.N + w) * kD;
  if (bad) {
    const float2 nan2 = make_float2(NAN, NAN);
    sk = nan2;
    sv = nan2;
    reinterpret_cast<float2*>(a.dq + o)[lane] = nan2;
  }
  reinterpret_cast<float2*>(a.dk + o)[lane] = sk;
  reinterpret_cast<float2*>(a.dv + o)[lane] = sv;
}

hipError_t launch_prefill_backward(const BwdArgs& a, int d, hipStream_t s) {
  if (d != kD || a.q_block != 128 || a.K > kListMaxB || a.K < 1) return hipErrorInvalidValue;
  if (a.levels < 1 || a.levels > 8 || a.N < 1 || a.nblk != (a.N + 127) / 128) return hipErrorInvalidValue;
  if ((int64_t)a.N * kRowB >= (1ll << 31) || (int64_t)a.Nc * kRowB >= (1ll << 31)) return hipErrorInvalidValue;
  if (a.R < (int64_t)a.N + (int64_t)a.nblk * a.K + 1 || a.R >= (1ll << 31)) return hipErrorInvalidValue;
  const int nh = a.B * a.H;
  if (nh == 0) return hipSuccess;
  const int64_t rows = (int64_t)nh * a.N;
  const int init_blocks = (int)std::min<int64_t>(8192, (rows * 64 + 255) / 256);
  hipLaunchKernelGGL(bwd_init_kernel, dim3(init_blocks), dim3(256), 0, s, a);
  int P = 2;
  while (P < a.K) P <<= 1;
  const size_t iv_lds = 3 * (size_t)P * sizeof(int32_t);
  if (iv_lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_interval_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)iv_lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_interval_kernel, dim3(a.nblk, nh), dim3(kIvThreads), iv_lds, s, a, P);
  hipLaunchKernelGGL(bwd_prefix_kernel, dim3(nh), dim3(kPxThreads), 0, s, a);
  const int hpx = (nh + 7) / 8;
  const dim3 units(8 * hpx * a.nblk);
  hipLaunchKernelGGL(bwd_dq_kernel, units, dim3(kDqThreads), 0, s, a);
  hipLaunchKernelGGL(bwd_dkv_kernel, units, dim3(kKvThreads), 0, s, a);
  if (a.Nc > 0) hipLaunchKernelGGL(bwd_reduce_coarse_kernel, dim3(a.Nc, nh), dim3(256), 0, s, a);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((a.N + 3) / 4, nh), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
