// Chunked prefill attention over pyramid-selected entries (Lighthouse
// summary, Methodology 2C: the chosen entries form a causally consistent
// subsequence, ordinary softmax attention runs on it, and each query's output
// goes back to its own position).
//
// For query block beta of one (sequence, head), query i = 128 beta + u sees
// the block's selected entries (rows of K/V for level 0, of the coarse K/V
// levels above) and the block's own level-0 keys 128 beta .. i (the lists
// and K/V belong to the head's KV head: GQA heads share both; a pyramid has
// one query head per KV head):
//   out[i] = sum_j softmax_j(q_i . k_j / sqrt(d)) v_j      (fp32)
// The coarse-query mode applies the same rule to the block's coarse query
// entries (2A: the pyramid is symmetric in Q, K and V): entry j of level l
// sees the block's list and the block's own level-l keys up to j, and its
// output goes to its own row of the output pyramid.
//
// gfx950 design, one 256-thread workgroup per (block, head), wave w owning
// queries 32w .. 32w+31:
//   * keys are processed in tiles of 32; the 256 threads gather K and V rows
//     by index straight from HBM into double-buffered LDS tiles, the loads
//     issued a step before they are staged.  K is kept row-major (rows padded
//     to 272 B), V transposed (d rows of 32 keys, padded to 72 B) - the
//     operand layouts the matrix cores want.
//   * a three-stage pipeline per step t: the scores of tile t+2 and the PV
//     product of tile t on the matrix cores, the softmax of tile t+1 on the
//     vector units, all independent, in one scheduling region.
//   * scores come out transposed, S^T = K Q^T (v_mfma_f32_16x16x32_bf16 with
//     the query block's fragments resident in registers), so every lane holds
//     8 keys x 2 queries; a query's running max is a reduction over 8 values
//     and 4 lanes.
//   * those probabilities are already the B operand of O^T = V^T P^T, so the
//     second product needs no data movement; P is split into a bf16 high part
//     and a bf16 remainder (two products) so the weights keep ~16 bits.
//   * blocks of a head run on one die: block ids are mapped so that each of
//     the 8 dies (round-robin dispatch) serves two heads, heaviest blocks
//     first, keeping the heads' selected rows hot in that die's L2.
#include <type_traits>

#include "args.hpp"
#include "common.hpp"

namespace sa {

typedef __bf16 bf16x8p __attribute__((ext_vector_type(8)));
typedef float f32x4p __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));

constexpr int kPfThreads = 256;
constexpr int kKT = 32;                 // keys per tile
constexpr int kD = 128;                 // head dim
constexpr int kKRow = kD + 8;           // K tile row stride (bf16 elements) = 272 B
constexpr int kVRow = 36;               // V^T tile row stride (bf16 elements) = 72 B
constexpr int kListMax = 8192;          // largest block_top_k the kernel stages in LDS
constexpr int kSeqMax = kListMax + 128 + 4 * kKT;   // + own keys + tail the gathers run past
constexpr uint32_t kCoarse = 0x80000000u;           // staged entry: coarse row flag
constexpr int kRowBytes = kD * 2;                   // one bf16 row of K or V
constexpr int kMaxRows = 1 << 23;                   // rows addressable by a staged byte offset
constexpr float kLazy = 8.f;            // log2 headroom before the softmax reference moves
// initial softmax reference: finite, so that a row with no visible key yet
// gives 2^(-inf - m) = 0 rather than 2^(-inf + inf)
constexpr float kMInit = -1e30f;

typedef float f32x2p __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2p __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 pair (round to nearest even, one instruction
// on gfx950), and the fp32 value of each half.
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2p){x, y}, bf16x2p));
}

// max of two or three scores as one instruction: fmaxf would first quiet
// each operand that the compiler cannot show to be canonical (a matrix-core
// result, a value that comes back from a lane swap), one extra instruction
// per operand; scores are never NaN
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max over the four lanes l16 + 16 jg (jg = 0..3) that hold one query's
// scores: a lane-swap across the wave's halves, then one across neighbouring
// 16-lane rows. Each swap exchanges half of its first operand with half of
// its second, so with both operands holding v, every lane ends with its own
// value in one result and its partner's in the other. The second operand is
// an opaque copy of v: given the same value twice, the compiler takes the
// two results as equal and keeps one of them.
__device__ __forceinline__ float max_over_lane_groups(float v) {
  uint32_t u = __float_as_uint(v), w = u;
  asm volatile("" : "+v"(w));
  auto r = __builtin_amdgcn_permlane32_swap(u, w, false, false);
  v = max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
  u = __float_as_uint(v);
  w = u;
  asm volatile("" : "+v"(w));
  r = __builtin_amdgcn_permlane16_swap(u, w, false, false);
  return max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Coarse-query mode: own entry u of a block whose level-0 part has nq rows
// starting at q0 (the block's level-1 entries first, then level 2, ...) ->
// its coarse row (-1 past the last), and in `first` the first own entry of
// its level.  Per-level tables are read with constant indices only.
__device__ __forceinline__ int coarse_entry(const PrefillArgs& a, int q0, int nq, int u, int& first) {
  int row = -1, acc = 0;
  first = 0;
#pragma unroll
  for (int l = 1; l < 8; ++l) {
    if (l < a.levels) {
      const int n = nq / a.c_span[l];
      if (row < 0 && u < acc + n) {
        row = a.c_off[l] + q0 / a.c_span[l] + (u - acc);
        first = acc;
      }
      acc += n;
    }
  }
  return row;
}

// coarse query entries of a block with nq level-0 rows
__device__ __forceinline__ int coarse_count(const PrefillArgs& a, int nq) {
  int acc = 0;
#pragma unroll
  for (int l = 1; l < 8; ++l)
    if (l < a.levels) acc += nq / a.c_span[l];
  return acc;
}

// HEADS = false: pyramid selection (each block's entry list from blk_idx,
// then the block's own keys).  HEADS = true: head-split prefill, no list:
// a block's key sequence is implicit - positions [0, A) (the sinks, A =
// min(sinks, end of block)) then [lo, end of block) (the window reaching
// back from the block's first query; everything for dense heads) - and each
// (query i, key j) pair is kept iff j <= i and (j < sinks or j > i - window).
template <bool HEADS>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kKT * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kD * kVRow];
  __shared__ __attribute__((aligned(16))) uint32_t s_seq[HEADS ? 4 : kSeqMax];

  int bh, kvh, blk;
  int S = 0, W = 0;                      // head-split: sinks and window of the head's class
  if constexpr (HEADS) {
    // ---- which (class, head, block): class 0 (the heavy dense heads) first;
    //      within a class die-major with a die's heads contiguous (the query
    //      heads of one KV head share a die's L2), heavy blocks first
    int L = blockIdx.x, cls = 0;
    if (L >= a.units0) { L -= a.units0; cls = 1; }
    const int nc = a.n_cls[cls];
    const int nbh = a.B * nc;
    const int hpx = (nbh + 7) / 8;
    const int xcd = L % 8, slot = L / 8;
    const int bi = xcd * hpx + slot % hpx;
    blk = a.nblk - 1 - slot / hpx;
    if (bi >= nbh || blk < 0) return;
    const int b = bi / nc, h = a.cls_heads[cls][bi - b * nc];
    bh = b * a.H + h;
    kvh = b * a.Hkv + h / a.G;
    if (cls == 0) { S = 0; W = a.N + 1; } else { S = a.sinks; W = a.window; }
  } else {
    // ---- which (head, block): die-major, heavy first; heads sharing a KV
    //      head (and its lists) on one die, otherwise two heads per die
    //      taken eight apart
    const int nh = a.B * a.H;
    const int hpx = (nh + 7) / 8;
    const int L = blockIdx.x;
    const int xcd = L % 8, slot = L / 8;
    bh = (a.G > 1) ? xcd * hpx + slot % hpx : xcd + 8 * (slot % hpx);
    blk = a.nblk - 1 - slot / hpx;
    if (bh >= nh || blk < 0) return;
    kvh = bh / a.G;
  }

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int l16 = lane & 15, jg = lane >> 4;
  const int q0 = blk * a.q_block;
  const int nq = min(a.q_block, a.N - q0);
  const int q1 = q0 + nq;
  int c_sel, T;
  int A = 0, lo = 0;                     // head-split: sink entries, first window position
  const int32_t* list = nullptr;
  if constexpr (HEADS) {
    A = min(S, q1);
    lo = (W > 0) ? max(A, q0 - W + 1) : q1;
    T = A + (q1 - lo);
    c_sel = 0;
  } else {
    c_sel = min(max(a.blk_count[(int64_t)kvh * a.nblk + blk], 0), min(a.K, kListMax));
    list = a.blk_idx + ((int64_t)kvh * a.nblk + blk) * a.K;
    T = c_sel + nq;
  }
  // queries of the tile: the block's level-0 rows, or (coarse mode) its
  // coarse entries, which are also its own keys after the list
  const bool coarse = !HEADS && a.coarse != 0;
  const int nqv = coarse ? coarse_count(a, nq) : nq;
  if (coarse) T = c_sel + nqv;
  const int ntiles = (T + kKT - 1) / kKT;
  const int64_t kv_rows = HEADS ? (int64_t)a.kv_stride : (int64_t)a.N;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)bh * a.N * kD;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k) + (int64_t)kvh * kv_rows * kD;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.v) + (int64_t)kvh * kv_rows * kD;
  const uint16_t* pkb = HEADS ? kb : reinterpret_cast<const uint16_t*>(a.pk) + (int64_t)kvh * a.Nc * kD;
  const uint16_t* pvb = HEADS ? vb : reinterpret_cast<const uint16_t*>(a.pv) + (int64_t)kvh * a.Nc * kD;
  // head-split: position of sequence entry e (e < T)
  auto pos = [&](int e) __attribute__((always_inline)) -> int { return e < A ? e : lo + (e - A); };
  // the row byte offset of sequence entry e: staged in LDS, or (head-split)
  // computed; past the end, row 0
  auto seq = [&](int e) __attribute__((always_inline)) -> uint32_t {
    if constexpr (HEADS) return (e < T) ? (uint32_t)pos(e) * kRowBytes : 0u;
    else return s_seq[e];
  };

  // ---- query fragments (B operand of S^T = K Q^T): query 32w + 16nt + l16,
  //      dims 32 jg + 8 s .. +8
  //      (coarse mode: the entry's row of pq, its coarse row in crow and the
  //      first own entry of its level in qlo; level-0 mode: qlo = 0)
  bf16x8p qf[2][4];
  int crow[2] = {0, 0}, qlo[2] = {0, 0};
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int ql = 32 * wid + 16 * nt + l16;
    const uint16_t* qrow = qb + (int64_t)(q0 + ql) * kD;
    if (coarse && ql < nqv) {
      crow[nt] = coarse_entry(a, q0, nq, ql, qlo[nt]);
      qrow = reinterpret_cast<const uint16_t*>(a.pq) + ((int64_t)bh * a.Nc + crow[nt]) * kD;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (ql < nqv) w = *reinterpret_cast<const uint4*>(qrow + 32 * jg + 8 * s);
      qf[nt][s] = __builtin_bit_cast(bf16x8p, w);
    }
  }

  // ---- the block's key sequence, staged once in LDS as row byte offsets:
  //      selected entry e < c_sel (a flat id: level-0 row, or coarse row
  //      flagged kCoarse), then the block's own level-0 keys q0 .. q0+nq-1,
  //      then row 0 for the tail that the gathers ahead run past (masked
  //      out of the softmax).  A flat id outside the pyramid is clamped to
  //      level-0 row 0 - never dereferenced out of bounds; its contribution
  //      is unspecified.
  if constexpr (!HEADS) {
    const int n_stage = (ntiles + 4) * kKT;
    for (int e = tid; e < n_stage; e += kPfThreads) {
      uint32_t r = 0u;
      if (e < c_sel) {
        const int f = list[e];
        if ((unsigned)f < (unsigned)a.N) r = (uint32_t)f * kRowBytes;
        else if ((unsigned)(f - a.N) < (unsigned)a.Nc) r = (uint32_t)(f - a.N) * kRowBytes | kCoarse;
      } else if (e < T) {
        if (coarse) {
          int first;
          r = (uint32_t)coarse_entry(a, q0, nq, e - c_sel, first) * kRowBytes | kCoarse;
        } else {
          r = (uint32_t)(q0 + e - c_sel) * kRowBytes;
        }
      }
      s_seq[e] = r;
    }
  }

  // ---- gather roles: K (thread -> key t/8, dims 8 (t%8) .. +8 and 64 + 8 (t%8)
  //      .. +8: the eight threads of a key write 128 contiguous bytes per
  //      store, which spreads them over all LDS banks), V (thread -> keys
  //      2(t%16), 2(t%16)+1, 8 dims at 8*(t/16)).
  const int gk_key = tid >> 3, gk_seg = tid & 7;
  const int gv_kp = tid & 15, gv_seg = tid >> 4;
  // a staged entry is a row's byte offset, the coarse flag in its top bit;
  // the bases already point at this thread's dims
  const char* k_seg = reinterpret_cast<const char*>(kb + 8 * gk_seg);
  const char* pk_seg = reinterpret_cast<const char*>(pkb + 8 * gk_seg);
  const char* v_seg = reinterpret_cast<const char*>(vb + 8 * gv_seg);
  const char* pv_seg = reinterpret_cast<const char*>(pvb + 8 * gv_seg);
  auto row_ptr = [](uint32_t r, const char* b0, const char* bc) -> const u32x4p* {
    const char* base = ((int32_t)r < 0) ? bc : b0;
    return reinterpret_cast<const u32x4p*>(base + (r & ~kCoarse));
  };
  // one set of loads for this thread: the K rows of tile x + 2 and the V rows
  // of tile x (K runs two tiles ahead: its scores are computed two tiles
  // before their PV product)
  struct Rows { u32x4p k0, k1, v0, v1; };
  // issue set x (unconditionally: past the end the rows are row 0, never used)
  auto gather = [&](int x, Rows& r) __attribute__((always_inline)) {
    const uint32_t lk = seq((x + 2) * kKT + gk_key);
    uint2 lv;
    if constexpr (HEADS) lv = make_uint2(seq(x * kKT + 2 * gv_kp), seq(x * kKT + 2 * gv_kp + 1));
    else lv = *reinterpret_cast<const uint2*>(&s_seq[x * kKT + 2 * gv_kp]);
    const u32x4p* pk = row_ptr(lk, k_seg, pk_seg);
    r.k0 = pk[0];
    r.k1 = pk[8];
    r.v0 = *row_ptr(lv.x, v_seg, pv_seg);
    r.v1 = *row_ptr(lv.y, v_seg, pv_seg);
  };
  auto stash_k = [&](int buf, const u32x4p& k0, const u32x4p& k1) __attribute__((always_inline)) {
    uint16_t* kdst = s_k[buf] + gk_key * kKRow + 8 * gk_seg;
    *reinterpret_cast<u32x4p*>(kdst) = k0;
    *reinterpret_cast<u32x4p*>(kdst + 64) = k1;
  };
  // set x: K of tile x + 2 into K buffer x & 1, V of tile x into V buffer
  // x & 1
  auto stash = [&](int x, const Rows& r) __attribute__((always_inline)) {
    stash_k(x & 1, r.k0, r.k1);
    const int buf = x & 1;
    // V^T: dims 8 gv_seg + i, keys 2 gv_kp and 2 gv_kp + 1 packed in one dword
    uint16_t* vdst = s_vt[buf] + (8 * gv_seg) * kVRow + 2 * gv_kp;
    auto put = [&](int i, uint32_t x0, uint32_t x1) __attribute__((always_inline)) {
      *reinterpret_cast<uint32_t*>(vdst + (2 * i) * kVRow) = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
      *reinterpret_cast<uint32_t*>(vdst + (2 * i + 1) * kVRow) = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
    };
    put(0, r.v0[0], r.v1[0]);
    put(1, r.v0[1], r.v1[1]);
    put(2, r.v0[2], r.v1[2]);
    put(3, r.v0[3], r.v1[3]);
  };

  // ---- running state for queries 32w + 16nt + l16
  float m[2] = {kMInit, kMInit}, lpart[2] = {0.f, 0.f};
  f32x4p o[8][2];                                   // O^T[d = 16 dt + 4 jg + i][q]
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) o[dt][nt] = (f32x4p){0.f, 0.f, 0.f, 0.f};
  const float sc = a.scale_log2;
  // packed bf16 pairs (-1, 0), (0, -1) and (1, 1) for the dot2 steps of the
  // softmax, held in registers: as instruction constants the compiler may
  // encode one as an inline float constant, which this instruction need not
  // read as the same pair
  uint32_t c_neg_lo = 0x0000BF80u, c_neg_hi = 0xBF800000u, c_ones = 0x3F803F80u;
  asm volatile("" : "+v"(c_neg_lo), "+v"(c_neg_hi), "+v"(c_ones));
  const bf16x2p neg_lo = __builtin_bit_cast(bf16x2p, c_neg_lo);
  const bf16x2p neg_hi = __builtin_bit_cast(bf16x2p, c_neg_hi);
  const bf16x2p ones = __builtin_bit_cast(bf16x2p, c_ones);

  // S^T[key = 16 mt + 4 jg + i][q = 16 nt + l16] of the tile in K buffer kbuf
  auto qk = [&](int kbuf, f32x4p (&s)[2][2]) __attribute__((always_inline)) {
    const uint16_t* kt = s_k[kbuf];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      bf16x8p kf[4];
#pragma unroll
      for (int st = 0; st < 4; ++st)
        kf[st] = __builtin_bit_cast(bf16x8p,
                                    *reinterpret_cast<const uint4*>(kt + (16 * mt + l16) * kKRow + 32 * jg + 8 * st));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4p c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[st], qf[nt][st], c, 0, 0, 0);
        s[mt][nt] = c;
      }
    }
  };

  // softmax of one tile's scores (log2 domain: p = 2^(s sc - m)) into its
  // P^T fragments: a bf16 high part and a bf16 remainder per query tile nt.
  // A query's reference m moves only when the tile's max exceeds it by more
  // than 2^8 (p stays <= 256, far from overflow); the factor 2^(m_old -
  // m_new) is returned in `alpha` (exactly 1 where m stays) and the caller
  // rescales the accumulators before it adds this tile's product, on a path
  // the whole wave skips when every factor is 1.  No branch in the common
  // case, so the caller's products and this vector work form one
  // scheduling region.  `mask` (a compile-time bool): the tile reaches past
  // the selection (causal mask over the block's own keys, nothing past the
  // end).
  struct PFrag { uint4 h[2], l[2]; };
  auto softmax = [&](auto mask, const int tile, f32x4p (&s)[2][2], PFrag& P,
                     float (&alpha)[2]) __attribute__((always_inline)) {
    if constexpr (decltype(mask)::value) {
      const int e0 = tile * kKT;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int ql = 32 * wid + 16 * nt + l16;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = e0 + 16 * mt + 4 * jg + i;
            bool ok;
            if constexpr (HEADS) {
              const int j = pos(e), qi = q0 + ql;
              ok = (e < T) & (j <= qi) & ((j < S) | (j > qi - W));
            } else {
              // bitwise, not short-circuit: one compare chain and one select
              const int u = e - c_sel;
              ok = (e < c_sel) | ((e < T) & (u <= ql) & (u >= qlo[nt]));
            }
            s[mt][nt][i] = ok ? s[mt][nt][i] : -INFINITY;
          }
      }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float t = max3_raw(s[0][nt][0], s[0][nt][1], s[0][nt][2]);
      t = max3_raw(t, s[0][nt][3], s[1][nt][0]);
      t = max3_raw(t, s[1][nt][1], s[1][nt][2]);
      const float mx = max_over_lane_groups(max_raw(t, s[1][nt][3])) * sc;
      const float mn = (mx - m[nt] > kLazy) ? mx : m[nt];
      alpha[nt] = __builtin_amdgcn_exp2f(m[nt] - mn);
      m[nt] = mn;
      lpart[nt] *= alpha[nt];
    }
    // the remainder p - hi(p) is exact in fp32 and comes from one dot2 of
    // the packed pair with (-1, 0) or (0, -1); the normaliser sums the two
    // bf16 parts (dot2 with (1, 1)), exactly the weights the product uses
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float p[8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p[4 * mt + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][nt][i], sc, -m[nt]));
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t h = pk_bf16(p[2 * j], p[2 * j + 1]);
        const bf16x2p hb = __builtin_bit_cast(bf16x2p, h);
        const float r0 = __builtin_amdgcn_fdot2_f32_bf16(hb, neg_lo, p[2 * j], false);
        const float r1 = __builtin_amdgcn_fdot2_f32_bf16(hb, neg_hi, p[2 * j + 1], false);
        hw[j] = h;
        lw[j] = pk_bf16(r0, r1);
        lpart[nt] = __builtin_amdgcn_fdot2_f32_bf16(hb, ones, lpart[nt], false);
        lpart[nt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2p, lw[j]), ones, lpart[nt], false);
      }
      P.h[nt] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      P.l[nt] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
  };
  // the rescale a softmax step asked for, before the next product
  auto rescale = [&](const float (&alpha)[2]) __attribute__((always_inline)) {
    if (__builtin_expect(!__all(alpha[0] == 1.f && alpha[1] == 1.f), 0)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) o[dt][nt] *= alpha[nt];
    }
  };

  // O^T += V^T P^T over one tile's 32 keys (V in buffer tile & 1): k-slot j
  // of lane group jg is key 4 jg + j (j < 4) or 16 + 4 jg + (j - 4)
  auto pv = [&](const int tile, const PFrag& P) __attribute__((always_inline)) {
    const uint16_t* vt = s_vt[tile & 1];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* vrow = vt + (16 * dt + l16) * kVRow;
      const uint2 w0 = *reinterpret_cast<const uint2*>(vrow + 4 * jg);
      const uint2 w1 = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * jg);
      const bf16x8p vf = __builtin_bit_cast(bf16x8p, make_uint4(w0.x, w0.y, w1.x, w1.y));
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(bf16x8p, P.h[nt]), o[dt][nt], 0, 0, 0);
        o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(bf16x8p, P.l[nt]), o[dt][nt], 0, 0, 0);
      }
    }
  };

  // one step of the pipeline at tile t: the scores of tile t + 2 and the PV
  // product of tile t go to the matrix cores while the vector units turn
  // the scores of tile t + 1 into its probabilities - the three are
  // independent, so one wave's vector work runs under its own products.
  // `mine` held set t (staged already) and now takes set t + 2; `next`
  // holds set t + 1, staged at the end.  s1 holds the scores of tile t + 1
  // and s2 receives those of tile t + 2; P0 holds the probabilities of tile
  // t and P1 receives those of tile t + 1.  Past the end the scores and
  // probabilities are of rows nobody reads (fully masked), so every step
  // runs the same instructions.
  float alpha[2];
  auto body = [&](auto mask, const int t, Rows& mine, const Rows& next, f32x4p (&s1)[2][2],
                  f32x4p (&s2)[2][2], const PFrag& P0, PFrag& P1) __attribute__((always_inline)) {
    rescale(alpha);
    gather(t + 2, mine);
    qk(t & 1, s2);
    pv(t, P0);
    softmax(mask, t + 1, s1, P1, alpha);
    stash(t + 1, next);
    lds_barrier();
  };

  // prologue: K of tiles 0 and 1 staged alone and their scores computed,
  // sets 0 and 1 in flight, tile 0's probabilities, then set 0 staged (its
  // K, of tile 2, over tile 0's once every wave has read those)
  lds_barrier();                                    // s_seq complete
  {
    const u32x4p* pk0 = row_ptr(seq(gk_key), k_seg, pk_seg);
    const u32x4p* pk1 = row_ptr(seq(kKT + gk_key), k_seg, pk_seg);
    stash_k(0, pk0[0], pk0[8]);
    stash_k(1, pk1[0], pk1[8]);
  }
  lds_barrier();
  f32x4p sa_[2][2], sb_[2][2];
  qk(0, sa_);
  qk(1, sb_);
  Rows ra, rb;
  gather(0, ra);
  gather(1, rb);
  PFrag pa, pb;
  const std::true_type masked;
  const std::false_type unmasked;
  softmax(masked, 0, sa_, pa, alpha);
  lds_barrier();                                    // K buffer 0 read by every wave
  stash(0, ra);
  lds_barrier();
  // pairs of tiles, then an odd last one: every path back to a loop head
  // passes both bodies of a pair, so the loads in flight there are always
  // set 1's.  Tiles from tile c_sel / 32 on reach past the selection: the
  // steps that turn them into probabilities take the masked form.
  int tile = 0;
  if constexpr (HEADS) {
    // tiles [0, u0) hold window entries that the block's last query does
    // not see (pos <= q1 - 1 - W), tiles from u1 on entries past the block's
    // first query (pos > q0) or past the sequence: both need the mask, the
    // tiles between do not (entries ascend in position)
    const int e_w = A + max(0, q1 - W - lo + 1);
    const int e_c = (q0 + 1 < A) ? q0 + 1 : A + max(0, q0 + 1 - lo);
    const int u0 = (min(e_w, T) + kKT - 1) / kKT;
    const int u1 = min(e_c, T) / kKT;
    for (; tile + 1 < ntiles && tile + 1 < u0; tile += 2) {
      body(masked, tile, ra, rb, sb_, sa_, pa, pb);
      body(masked, tile + 1, rb, ra, sa_, sb_, pb, pa);
    }
    for (; tile + 2 < u1; tile += 2) {
      body(unmasked, tile, ra, rb, sb_, sa_, pa, pb);
      body(unmasked, tile + 1, rb, ra, sa_, sb_, pb, pa);
    }
    for (; tile + 1 < ntiles; tile += 2) {
      body(masked, tile, ra, rb, sb_, sa_, pa, pb);
      body(masked, tile + 1, rb, ra, sa_, sb_, pb, pa);
    }
  } else {
    const int mask_from = c_sel / kKT;
    for (; tile + 2 < mask_from; tile += 2) {
      body(unmasked, tile, ra, rb, sb_, sa_, pa, pb);
      body(unmasked, tile + 1, rb, ra, sa_, sb_, pb, pa);
    }
    for (; tile + 1 < ntiles; tile += 2) {
      body(masked, tile, ra, rb, sb_, sa_, pa, pb);
      body(masked, tile + 1, rb, ra, sa_, sb_, pb, pa);
    }
  }
  if (tile < ntiles) body(masked, tile, ra, rb, sb_, sa_, pa, pb);
  rescale(alpha);

  // ---- normalise and write: lane holds d = 16 dt + 4 jg + 0..3 of query
  //      32w + 16 nt + l16
  float* ob = a.out + (int64_t)bh * a.N * kD;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float lt = lpart[nt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int ql = 32 * wid + 16 * nt + l16;
    if (ql < nqv) {
      // the row's log-sum-exp (natural log) for the backward pass: the
      // weights were 2^(s sc - m), so the denominator is 2^m lt
      if (a.lse != nullptr && !coarse && jg == 0)
        a.lse[(int64_t)bh * a.N + q0 + ql] = (m[nt] + log2f(lt)) * 0.6931471805599453f;
      const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
      // the scatter back: a level-0 query's own row, or the coarse entry's
      // own row of the output pyramid
      float* orow = coarse ? a.out_c + ((int64_t)bh * a.Nc + crow[nt]) * kD
                           : ob + (int64_t)(q0 + ql) * kD;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4p v = o[dt][nt] * inv;
        *reinterpret_cast<float4*>(orow + 16 * dt + 4 * jg) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

hipError_t launch_prefill(const PrefillArgs& a, int d, hipStream_t s) {
  if (d != kD || a.q_block != 128 || a.K > kListMax) return hipErrorInvalidValue;
  if (a.G < 1 || a.H != a.Hkv * a.G || (a.G > 1 && a.Nc > 0)) return hipErrorInvalidValue;
  if (a.N >= kMaxRows || a.Nc >= kMaxRows) return hipErrorInvalidValue;
  if (a.coarse) {
    // the block's coarse entries fit one query tile (sum of 128 / p^l < 128)
    // and every level's spans tile the block
    if (a.levels < 2 || a.levels > 8 || !a.pq || !a.out_c || a.Nc < 1) return hipErrorInvalidValue;
    int n = 0;
    for (int l = 1; l < a.levels; ++l) {
      if (a.c_span[l] < 2 || a.q_block % a.c_span[l] || a.N % a.c_span[l]) return hipErrorInvalidValue;
      n += a.q_block / a.c_span[l];
    }
    if (n > 128) return hipErrorInvalidValue;
  }
  const int nh = a.B * a.H;
  const int hpx = (nh + 7) / 8;
  dim3 grid(8 * hpx * a.nblk);
  hipLaunchKernelGGL(prefill_kernel<false>, grid, dim3(kPfThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_heads(const PrefillArgs& a, int d, hipStream_t s) {
  if (d != kD || a.q_block != 128 || a.G < 1 || a.H != a.Hkv * a.G) return hipErrorInvalidValue;
  if (a.N >= kMaxRows || a.kv_stride < a.N) return hipErrorInvalidValue;
  int units = 0;
  for (int c = 0; c < 2; ++c) {
    if (a.n_cls[c] < 0 || a.n_cls[c] > kMaxPrefillHeads) return hipErrorInvalidValue;
    for (int i = 0; i < a.n_cls[c]; ++i)
      if (a.cls_heads[c][i] >= a.H) return hipErrorInvalidValue;
    const int u = 8 * ((a.B * a.n_cls[c] + 7) / 8) * a.nblk;
    if (c == 0 && u != a.units0) return hipErrorInvalidValue;
    units += u;
  }
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_kernel<true>, dim3(units), dim3(kPfThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
