// Joint top-K across pyramid levels for every block of queries (Lighthouse
// summary, Methodology 2B: a blockwise top-K picks entries across all levels
// jointly; 2C: the chosen entries must form a causally consistent set).
//
// Block beta of q_block level-0 queries may use entry (l, j) of level l when
// its span ends before the block starts: (j + 1) * p^l <= q_block * beta.  The
// visible entries of every level are therefore a prefix, and among them the K
// with the largest score are kept, ties going to the lower level and then the
// lower index - which is the order of the flat entry ids off_l + j.  When at
// most K entries are visible, all are kept.
//
// The K-th largest score key (the cut) is resolved by radix levels of up to
// 12 bits over LDS histograms, with no sort; the digits start below the
// leading bits all keys of the head share (an AND/OR reduction over the head,
// one small launch first), so the buckets are well spread.  The kept flat ids
// are written in ascending order (strictly larger keys, then the first ties by
// flat id).
//
// Visibility only grows with the block index, so the cut never decreases
// along a head's blocks.  Blocks are grouped into intervals of S: one
// workgroup per interval resolves the cut of the interval's first block over
// its visible prefixes - a lower bound of every later block's cut - and
// stores, in ascending flat id, the entries the interval's last block sees
// whose key reaches that bound (the kept entries of every block in the
// interval are among them; about K + S x (entries a block adds)).  Each block
// then selects from its visible candidates in LDS instead of passing over all
// its visible scores.  An interval with more than kPsCap candidates (many
// equal scores) leaves its blocks to the full passes.
#include "args.hpp"
#include "common.hpp"

namespace sa {

constexpr int kPsThreads = 256;

struct VisRanges {
  int nl;
  int64_t off[8];     // flat id of the level's first entry
  int cnt[8];         // visible entries of the level
  int64_t total;
};

__device__ __forceinline__ VisRanges visible(const PyrSelectArgs& a, int blk) {
  VisRanges v;
  v.nl = a.levels;
  v.total = 0;
  int width = 1;
  for (int l = 0; l < 8; ++l) {
    if (l >= a.levels) { v.off[l] = 0; v.cnt[l] = 0; continue; }
    const int len = a.len[l];
    const int c = (int)min((int64_t)len, (int64_t)a.q_block * blk / width);
    v.off[l] = a.soff[l];
    v.cnt[l] = c;
    v.total += c;
    width *= a.factor;
  }
  return v;
}

constexpr int kPsU = 16;                 // entries per thread in flight per pass step

// key >> pos for pos in 0..32 (a 32-bit shift by 32 is not defined)
__device__ __forceinline__ uint32_t key_hi(uint32_t key, int pos) { return pos >= 32 ? 0u : key >> pos; }

// AND and OR of every score key of one (sequence, head): the leading bits
// all its keys share.  One 1024-thread workgroup per head.
__global__ __launch_bounds__(1024) void pyr_prefix_kernel(PyrSelectArgs a) {
  __shared__ uint32_t s_and[16], s_or[16];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* sc = a.scores + (int64_t)bh * a.Nt;
  uint32_t kand = 0xFFFFFFFFu, kor = 0u;
  for (int j0 = 0; j0 < a.Nt; j0 += 1024 * kPsU) {
    float x[kPsU];
#pragma unroll
    for (int u = 0; u < kPsU; ++u) {
      const int j = j0 + u * 1024 + tid;
      x[u] = sc[j < a.Nt ? j : a.Nt - 1];
    }
#pragma unroll
    for (int u = 0; u < kPsU; ++u) {
      const uint32_t key = order_key(x[u]);
      kand &= key;
      kor |= key;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    kand &= (uint32_t)__shfl_xor((int)kand, m);
    kor |= (uint32_t)__shfl_xor((int)kor, m);
  }
  if ((tid & 63) == 0) { s_and[tid >> 6] = kand; s_or[tid >> 6] = kor; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 16; ++w) { kand &= s_and[w]; kor |= s_or[w]; }
    a.prefix[bh] = make_uint2(kand, kor);
  }
}

// Histogram of the visible keys whose bits above `pshift` equal `prefix`,
// bucket = (key >> shift) & (2^bits - 1).  Each thread keeps kPsU loads in
// flight, and the next chunk's loads are issued before a chunk is counted.
template <int NT>
__device__ void vis_hist(const float* sc, const VisRanges& v, uint32_t prefix, int pshift, int shift,
                         int bits, uint32_t* hist) {
  const uint32_t mask = (1u << bits) - 1u;
  for (int l = 0; l < v.nl; ++l) {
    const float* p = sc + v.off[l];
    const int cnt = v.cnt[l];
    if (cnt <= 0) continue;
    auto load = [&](float (&x)[kPsU], int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kPsU; ++u) {
        const int j = j0 + u * NT + threadIdx.x;
        x[u] = p[j < cnt ? j : cnt - 1];
      }
    };
    auto count = [&](const float (&x)[kPsU], int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kPsU; ++u) {
        const int j = j0 + u * NT + threadIdx.x;
        const uint32_t key = order_key(x[u]);
        if (j < cnt && key_hi(key, pshift) == prefix)
          atomicAdd(&hist[(key >> shift) & mask], 1u);
      }
    };
    float xa[kPsU], xb[kPsU];
    load(xa, 0);
    for (int j0 = 0; j0 < cnt; j0 += 2 * kPsU * NT) {
      load(xb, j0 + kPsU * NT);
      count(xa, j0);
      if (j0 + kPsU * NT >= cnt) break;
      load(xa, j0 + 2 * kPsU * NT);
      count(xb, j0 + kPsU * NT);
    }
  }
}

// Scan a histogram of NB buckets from the top for the bucket holding the
// `target`-th key; returns the bucket and adds the count above it to *above.
template <int NB, int NT>
__device__ int vis_find(const uint32_t* hist, int64_t target, int64_t* above, int64_t* s_scan,
                        int* s_b, int64_t* s_above) {
  constexpr int PER = NB / NT;
  const int tid = threadIdx.x;
  int64_t tc = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) tc += hist[NB - 1 - (PER * tid + k)];
  int64_t tot;
  const int64_t pre = block_exclusive_scan<int64_t, NT>(tc, s_scan, &tot);
  if (tid == 0) *s_b = -1;
  __syncthreads();
  int64_t cc = *above + pre;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int bk = NB - 1 - (PER * tid + k);
    const int64_t nc = cc + hist[bk];
    if (hist[bk] && cc < target && nc >= target) { *s_b = bk; *s_above = cc; }
    cc = nc;
  }
  __syncthreads();
  const int b = *s_b;
  *above = *s_above;
  __syncthreads();
  return b;
}

struct PsShared {
  uint32_t hist[4096];
  int64_t scan[16];                  // one entry per wave, up to 1024 threads
  uint32_t scan32[16];
  int b;
  int64_t above;
  uint32_t kand[16], kor[16];
  uint32_t n;
};

// The cut over the visible prefixes v of one head: the key of the K-th
// largest visible score; *above receives how many visible keys exceed it.
template <int NT>
__device__ uint32_t visible_cut(const PyrSelectArgs& a, const VisRanges& v, const float* sc, int bh,
                                PsShared& sh, int64_t* above_out, int64_t target) {
  const uint2 pf = a.prefix[bh];
  const uint32_t diff = pf.x ^ pf.y;
  const int common = diff ? __clz(diff) : 32;
  int64_t above = 0;
  uint32_t cut = pf.x;                              // when every key is equal
  if (common < 32) {
    int pos = 32 - common;                          // bits still to resolve
    uint32_t prefix = key_hi(pf.x, pos);
    while (pos > 0) {                               // digits of at most 12 bits
      const int bits = pos < 12 ? pos : 12;
      const int shift = pos - bits;
      for (int i = threadIdx.x; i < 4096; i += NT) sh.hist[i] = 0;
      __syncthreads();
      vis_hist<NT>(sc, v, prefix, pos, shift, bits, sh.hist);
      __syncthreads();
      const int bk = vis_find<4096, NT>(sh.hist, target, &above, sh.scan, &sh.b, &sh.above);
      prefix = (prefix << bits) | (uint32_t)bk;
      pos = shift;
    }
    cut = prefix;
  }
  *above_out = above;
  return cut;
}

// Every visible key at least lb, gathered into keys[0, cap) in no particular
// order (one LDS atomic per wave and load step); returns how many there are
// (all are counted, the first cap stored).
template <int NT>
__device__ uint32_t collect_at_least(const float* sc, const VisRanges& v, uint32_t lb, uint32_t* keys,
                                     int cap, uint32_t* s_n) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x == 0) *s_n = 0;
  __syncthreads();
  for (int l = 0; l < v.nl; ++l) {
    const float* p = sc + v.off[l];
    const int cnt = v.cnt[l];
    if (cnt <= 0) continue;
    auto load = [&](float (&x)[kPsU], int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kPsU; ++u) {
        const int j = j0 + u * NT + threadIdx.x;
        x[u] = p[j < cnt ? j : cnt - 1];
      }
    };
    auto put = [&](const float (&x)[kPsU], int j0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kPsU; ++u) {
        const int j = j0 + u * NT + threadIdx.x;
        const uint32_t key = order_key(x[u]);
        const bool keep = j < cnt && key >= lb;
        const uint64_t m = __ballot(keep);
        if (m) {
          uint32_t base = 0;
          if (lane == 0) base = atomicAdd(s_n, (uint32_t)__popcll(m));
          base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
          const uint32_t pos = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (keep && pos < (uint32_t)cap) keys[pos] = key;
        }
      }
    };
    float xa[kPsU], xb[kPsU];
    load(xa, 0);
    for (int j0 = 0; j0 < cnt; j0 += 2 * kPsU * NT) {
      load(xb, j0 + kPsU * NT);
      put(xa, j0);
      if (j0 + kPsU * NT >= cnt) break;
      load(xa, j0 + 2 * kPsU * NT);
      put(xb, j0 + kPsU * NT);
    }
  }
  __syncthreads();
  return *s_n;
}

// Ordered compaction of the scores p[0, cnt) whose key is at least tau: each
// goes to emit(slot, key, id = base + index), slots in index order. Thread t
// takes kPsU consecutive entries of every chunk; the next chunk's loads are
// issued before a chunk is scanned. Returns the count.
template <int NT, typename Emit>
__device__ uint32_t compact_scores(const float* p, int cnt, int base, uint32_t tau, Emit emit,
                                   uint32_t* s_scan32) {
  if (cnt <= 0) return 0;
  uint32_t run = 0;
  auto load = [&](float (&x)[kPsU], int j0) __attribute__((always_inline)) {
    const int jt = j0 + kPsU * (int)threadIdx.x;
#pragma unroll
    for (int u = 0; u < kPsU; ++u) x[u] = p[min(jt + u, cnt - 1)];
  };
  auto step = [&](const float (&x)[kPsU], int j0) __attribute__((always_inline)) {
    const int jt = j0 + kPsU * (int)threadIdx.x;
    uint32_t f = 0;
#pragma unroll
    for (int u = 0; u < kPsU; ++u)
      if (jt + u < cnt && order_key(x[u]) >= tau) f |= 1u << u;
    uint32_t tot;
    uint32_t o = run + block_exclusive_scan<uint32_t, NT>(__popc(f), s_scan32, &tot);
#pragma unroll
    for (int u = 0; u < kPsU; ++u)
      if (f & (1u << u)) emit(o++, order_key(x[u]), base + jt + u);
    run += tot;
  };
  float xa[kPsU], xb[kPsU];
  load(xa, 0);
  for (int j0 = 0; j0 < cnt; j0 += 2 * kPsU * NT) {
    load(xb, j0 + kPsU * NT);
    step(xa, j0);
    if (j0 + kPsU * NT >= cnt) break;
    load(xa, j0 + 2 * kPsU * NT);
    step(xb, j0 + kPsU * NT);
  }
  return run;
}

// The cut over n keys held in LDS, as visible_cut does over global prefixes,
// given that it lies in [lo, hi]: the keys above hi are counted (all above
// the cut), and the radix digits run below the bits lo and hi share - the
// keys in the window spread over the buckets even when a few keys far above
// it (outliers) would otherwise crowd the bulk into one bucket.
template <int NT>
__device__ uint32_t lds_cut(const uint32_t* keys, int n, int64_t K, uint32_t lo, uint32_t hi,
                            PsShared& sh, int64_t* above_out) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t over = 0;
  for (int i = tid; i < n; i += NT) over += keys[i] > hi ? 1u : 0u;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) over += (uint32_t)__shfl_xor((int)over, m);
  if (lane == 0) sh.kand[tid >> 6] = over;
  __syncthreads();
  int64_t above = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) above += sh.kand[w];
  const uint32_t diff = lo ^ hi;
  const int common = diff ? __clz(diff) : 32;
  uint32_t cut = lo;                               // lo == hi: the window is one key
  if (common < 32) {
    int pos = 32 - common;
    uint32_t prefix = key_hi(lo, pos);
    while (pos > 0) {
      const int bits = pos < 12 ? pos : 12;
      const int shift = pos - bits;
      const uint32_t mask = (1u << bits) - 1u;
      for (int i = tid; i < 4096; i += NT) sh.hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        const uint32_t key = keys[i];
        if (key <= hi && key_hi(key, pos) == prefix) atomicAdd(&sh.hist[(key >> shift) & mask], 1u);
      }
      __syncthreads();
      const int bk = vis_find<4096, NT>(sh.hist, K, &above, sh.scan, &sh.b, &sh.above);
      prefix = (prefix << bits) | (uint32_t)bk;
      pos = shift;
    }
    cut = prefix;
  }
  *above_out = above;
  return cut;
}

// One workgroup per (interval, sequence-head): the cut of the interval's first
// block, then the candidates of the interval (entries its last block sees with
// a key at least that cut).
constexpr int kPiThreads = 256;

// Workgroup ids are dealt to the 8 dies round-robin. The interval kernels
// renumber them so that each die takes whole heads: the passes over a head's
// scores then hit that die's own L2. Within a head, late intervals (they see
// the most entries) come first.
__device__ __forceinline__ void die_major(int n_int, int nbh, int* iv, int* bh) {
  const int total = n_int * nbh;
  const int L = (int)blockIdx.x, x = L & 7, j = L >> 3;
  const int q = total >> 3, r = total & 7;
  const int idx = x * q + min(x, r) + j;
  *bh = idx / n_int;
  *iv = n_int - 1 - (idx - *bh * n_int);
}

__global__ __launch_bounds__(kPiThreads) void pyr_interval_kernel(PyrSelectArgs a) {
  __shared__ PsShared sh;
  __shared__ uint32_t c_key[kPsCap];
  int iv, bh;
  die_major(a.n_int, a.B * a.H, &iv, &bh);
  const int tid = threadIdx.x;
  const int b0 = iv * a.S, b1 = min(b0 + a.S, a.nblk) - 1;
  const int64_t slot = (int64_t)bh * a.n_int + iv;
  const VisRanges v1 = visible(a, b1);
  if (v1.total <= a.K) {                    // every block of the interval keeps all it sees
    if (tid == 0) { a.tau[slot] = 0; a.tau_hi[slot] = 0; a.cand_len[slot] = 0; }
    return;
  }
  const float* sc = a.scores + (int64_t)bh * a.Nt;
  const VisRanges v0 = visible(a, b0);
  uint32_t tau = 0;
  if (v0.total > a.K) {
    // A lower bound first: a visible entry of the top level carries its
    // score down a chain of one entry per level (the child holding its max),
    // all visible and all with that score, so the ceil(K/L)-th largest
    // visible top-level score has at least K visible entries at or above it.
    // The keys reaching the bound are gathered in LDS and the exact cut taken
    // there; with too many of them (or too few top-level entries) the radix
    // passes run over every visible score.
    int64_t above;
    bool done = false;
    const int L = v0.nl;
    const int64_t tk = (a.K + L - 1) / L;
    if (L > 1 && v0.cnt[L - 1] >= tk) {
      VisRanges vt = v0;
      for (int l = 0; l < L - 1; ++l) vt.cnt[l] = 0;
      vt.total = v0.cnt[L - 1];
      const uint32_t lb = visible_cut<kPiThreads>(a, vt, sc, bh, sh, &above, tk);
      const uint32_t n = collect_at_least<kPiThreads>(sc, v0, lb, c_key, kPsCap, &sh.n);
      if (n <= (uint32_t)kPsCap) {
        tau = lds_cut<kPiThreads>(c_key, (int)n, a.K, lb, 0xFFFFFFFFu, sh, &above);
        done = true;
      }
      __syncthreads();
    }
    if (!done) tau = visible_cut<kPiThreads>(a, v0, sc, bh, sh, &above, a.K);
  }
  uint2* out = a.cand + slot * kPsCap;
  uint32_t total = 0;
  for (int l = 0; l < v1.nl; ++l) {
    const float* p = sc + v1.off[l];
    const int base = (int)v1.off[l];
    const uint32_t room = total < (uint32_t)kPsCap ? (uint32_t)kPsCap - total : 0u;
    uint2* o = out + min(total, (uint32_t)kPsCap);
    total += compact_scores<kPiThreads>(
        p, v1.cnt[l], base, tau,
        [&](uint32_t k, uint32_t key, int32_t id) {
          if (k < room) {
            o[k] = make_uint2(key, (uint32_t)id);
            c_key[(o - out) + k] = key;
          }
        },
        sh.scan32);
  }
  // the last block's cut, over the candidates (they hold every entry it
  // keeps): an upper bound of the cut of every block in the interval
  uint32_t tau_hi = 0xFFFFFFFFu;
  if (total <= (uint32_t)kPsCap) {
    __syncthreads();
    int64_t above;
    tau_hi = lds_cut<kPiThreads>(c_key, (int)total, a.K, tau, 0xFFFFFFFFu, sh, &above);
  }
  if (tid == 0) {
    a.tau[slot] = tau;
    a.tau_hi[slot] = tau_hi;
    a.cand_len[slot] = total <= (uint32_t)kPsCap ? (int32_t)total : -1;
  }
}

// One block's selection by whole-workgroup passes over its visible scores:
// every visible entry when at most K are visible, else the cut and the kept
// flat ids in ascending order (strict, then the first ties).
template <int NT>
__device__ __forceinline__ void full_select(const PyrSelectArgs& a, int blk, int bh, PsShared& sh) {
  const int tid = threadIdx.x;
  const VisRanges v = visible(a, blk);
  const float* sc = a.scores + (int64_t)bh * a.Nt;
  int32_t* out = a.blk_idx + ((int64_t)bh * a.nblk + blk) * a.K;
  const int64_t K = a.K;
  if (v.total <= K) {                      // every visible entry
    int64_t o = 0;
    for (int l = 0; l < v.nl; ++l) {
      for (int j = tid; j < v.cnt[l]; j += NT) out[o + j] = (int32_t)(v.off[l] + j);
      o += v.cnt[l];
    }
    if (tid == 0) a.blk_count[(int64_t)bh * a.nblk + blk] = (int32_t)v.total;
    return;
  }
  int64_t above;
  const uint32_t cut = visible_cut<NT>(a, v, sc, bh, sh, &above, a.K);
  const uint32_t need = (uint32_t)(K - above);        // ties kept, lowest flat ids first

  // ascending flat ids: strict (key > cut) and the first `need` ties; thread
  // t takes kPsU consecutive entries of each chunk, loaded together
  uint32_t s_run = 0, t_run = 0;                      // totals of earlier chunks
  for (int l = 0; l < v.nl; ++l) {
    const float* p = sc + v.off[l];
    const int cnt = v.cnt[l];
    for (int j0 = 0; j0 < cnt; j0 += kPsU * NT) {
      const int jt = j0 + kPsU * tid;
      float x[kPsU];
#pragma unroll
      for (int u = 0; u < kPsU; ++u) x[u] = p[(jt + u) < cnt ? jt + u : cnt - 1];
      uint32_t sf = 0, tf = 0;
#pragma unroll
      for (int u = 0; u < kPsU; ++u) {
        const uint32_t key = order_key(x[u]);
        if (jt + u < cnt) {
          if (key > cut) sf |= 1u << u;
          else if (key == cut) tf |= 1u << u;
        }
      }
      uint32_t tot_s, tot_t;
      const uint32_t ex_s = block_exclusive_scan<uint32_t, NT>(__popc(sf), sh.scan32, &tot_s);
      const uint32_t ex_t = block_exclusive_scan<uint32_t, NT>(__popc(tf), sh.scan32, &tot_t);
      uint32_t sb = s_run + ex_s, tb = t_run + ex_t;
#pragma unroll
      for (int u = 0; u < kPsU; ++u) {
        if (sf & (1u << u)) {
          out[sb + (tb < need ? tb : need)] = (int32_t)(v.off[l] + jt + u);
          ++sb;
        } else if (tf & (1u << u)) {
          if (tb < need) out[sb + tb] = (int32_t)(v.off[l] + jt + u);
          ++tb;
        }
      }
      s_run += tot_s;
      t_run += tot_t;
    }
  }
  if (tid == 0) a.blk_count[(int64_t)bh * a.nblk + blk] = (int32_t)K;
}

// Without intervals: one workgroup per (block, sequence-head), late blocks
// (the most visible entries) first.
__global__ __launch_bounds__(kPsThreads) void pyr_select_kernel(PyrSelectArgs a) {
  __shared__ PsShared sh;
  full_select<kPsThreads>(a, a.nblk - 1 - (int)blockIdx.x, blockIdx.y, sh);
}

// ---------------------------------------------------------------- one wave per block
// With intervals, one workgroup per (interval, sequence-head) stages the
// interval's candidates in LDS once, and each wave selects for its own blocks
// of the interval with no workgroup barrier:
//  * the candidates are in ascending flat id and each level's visible entries
//    are a prefix of the level, so a block's visible candidates are one range
//    per level, found by a search;
//  * the cut lies between the interval's two bounds: keys above the upper one
//    are counted, and radix digits of 8 bits below the bits the bounds share
//    go through a 256-bucket histogram of the wave's own;
//  * the kept ids are written in ascending flat id, positions from ballots.
// An interval with more candidates than fit runs the whole-workgroup passes
// for each of its blocks.
constexpr int kPwWaves = 8;
constexpr int kPwThreads = kPwWaves * 64;
constexpr int kPwBuckets = 256;

union PwShared {
  struct {
    uint32_t key[kPsCap];
    int32_t id[kPsCap];
    uint32_t hist[kPwWaves][kPwBuckets];
  } w;
  PsShared ps;
};

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

// lanes below this one whose bit is set in m
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// First index i in ids[0, n) (ascending) with ids[i] >= x, by the whole wave:
// 64 segments tested at their last element, then the one segment holding the
// boundary element by element.
__device__ int wave_lower_bound(const int32_t* ids, int n, int64_t x, int lane) {
  if (n == 0) return 0;
  const int seg = (n + 63) / 64;
  const int last = min((lane + 1) * seg, n) - 1;
  const bool below = lane * seg < n && ids[last] < x;
  const int j = __popcll(wave_ballot(below));          // segments wholly below x
  if (j * seg >= n) return n;
  int cnt = 0;
  for (int t0 = 0; t0 < seg; t0 += 64) {
    const int i = j * seg + t0 + lane;
    cnt += __popcll(wave_ballot(t0 + lane < seg && i < n && ids[i] < x));
  }
  return j * seg + cnt;
}

// A bucket of hist[0, 256) counted from the top: the one holding the
// target-th key when `above` keys lie above the histogram. Returns it and
// adds the count above it to *above.
__device__ int wave_find256(const uint32_t* hist, uint32_t target, uint32_t* above, int lane) {
  uint32_t c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) c[k] = hist[kPwBuckets - 1 - 4 * lane - k];
  const uint32_t sum = c[0] + c[1] + c[2] + c[3];
  const uint32_t incl = wave_inclusive_scan(sum);
  uint32_t base = *above + incl - sum;
  const uint64_t m = wave_ballot(base < target && target <= base + sum);
  const int src = m ? (int)__builtin_ctzll(m) : 0;            // m != 0 while target <= the total
  int bk = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (bk == 0 && base + c[k] >= target) bk = kPwBuckets - 4 * lane - k;   // bucket + 1
    else if (bk == 0) base += c[k];
  }
  const int b = __builtin_amdgcn_readlane(bk, src) - 1;
  *above = (uint32_t)__builtin_amdgcn_readlane((int)base, src);
  return b;
}

// wave-local ordering of LDS accesses (one wave's own histogram)
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

struct LevelRanges { int lo[8]; };

__device__ __forceinline__ void wave_select(const PyrSelectArgs& a, const PwShared& s, uint32_t* hist,
                                            int ncand, const LevelRanges lstart, int blk, int bh,
                                            uint32_t lo, uint32_t hi, int lane) {
  const VisRanges v = visible(a, blk);
  int32_t* out = a.blk_idx + ((int64_t)bh * a.nblk + blk) * a.K;
  const uint32_t K = (uint32_t)a.K;
  if (v.total <= (int64_t)K) {
    int64_t o = 0;
#pragma unroll
    for (int l = 0; l < 8; ++l) {
      if (l < v.nl) {
        for (int j = lane; j < v.cnt[l]; j += 64) out[o + j] = (int32_t)(v.off[l] + j);
        o += v.cnt[l];
      }
    }
    if (lane == 0) a.blk_count[(int64_t)bh * a.nblk + blk] = (int32_t)v.total;
    return;
  }
  // the visible candidates: [lstart.lo[l], lend[l]) of each level (the
  // level loops are unrolled so that the bounds stay in registers)
  int lend[8];
#pragma unroll
  for (int l = 0; l < 8; ++l)
    lend[l] = l < v.nl ? wave_lower_bound(s.w.id, ncand, v.off[l] + v.cnt[l], lane) : 0;
  // keys above the upper bound: all kept
  uint32_t over = 0;
#pragma unroll
  for (int l = 0; l < 8; ++l)
    if (l < v.nl)
      for (int i = lstart.lo[l] + lane; i < lend[l]; i += 64) over += s.w.key[i] > hi ? 1u : 0u;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) over += (uint32_t)__shfl_xor((int)over, m);
  uint32_t above = over;
  const uint32_t diff = lo ^ hi;
  const int common = diff ? __clz(diff) : 32;
  uint32_t cut = lo;                                   // lo == hi: the window is one key
  if (common < 32) {
    int pos = 32 - common;
    uint32_t prefix = key_hi(lo, pos);
    while (pos > 0) {
      const int bits = pos < 8 ? pos : 8;
      const int shift = pos - bits;
      const uint32_t mask = (1u << bits) - 1u;
#pragma unroll
      for (int k = 0; k < 4; ++k) hist[4 * lane + k] = 0;
      wave_lds_sync();
#pragma unroll
      for (int l = 0; l < 8; ++l)
        if (l < v.nl)
          for (int i = lstart.lo[l] + lane; i < lend[l]; i += 64) {
            const uint32_t key = s.w.key[i];
            if (key <= hi && key_hi(key, pos) == prefix) atomicAdd(&hist[(key >> shift) & mask], 1u);
          }
      wave_lds_sync();
      const int bk = wave_find256(hist, K, &above, lane);
      wave_lds_sync();
      prefix = (prefix << bits) | (uint32_t)bk;
      pos = shift;
    }
    cut = prefix;
  }
  const uint32_t need = K - above;                     // ties kept, lowest flat ids first
  // every position is below K when `above` counts the keys over the cut;
  // the test keeps a write inside the block's K slots regardless
  uint32_t srun = 0, trun = 0;
#pragma unroll
  for (int l = 0; l < 8; ++l)
    if (l < v.nl)
      for (int i0 = lstart.lo[l]; i0 < lend[l]; i0 += 64) {
        const int i = i0 + lane;
        const bool ok = i < lend[l];
        const uint32_t key = ok ? s.w.key[i] : 0u;
        const bool st = ok && key > cut, ti = ok && key == cut;
        const uint64_t ms = wave_ballot(st), mt = wave_ballot(ti);
        const uint32_t sb = srun + lanes_below(ms), tb = trun + lanes_below(mt);
        const uint32_t p = st ? sb + (tb < need ? tb : need) : sb + tb;
        if ((st || (ti && tb < need)) && p < K) out[p] = s.w.id[i];
        srun += (uint32_t)__popcll(ms);
        trun += (uint32_t)__popcll(mt);
      }
  if (lane == 0) a.blk_count[(int64_t)bh * a.nblk + blk] = (int32_t)K;
}

__global__ __launch_bounds__(kPwThreads) void pyr_block_select_kernel(PyrSelectArgs a) {
  __shared__ PwShared s;
  int iv, bh;
  die_major(a.n_int, a.B * a.H, &iv, &bh);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t slot = (int64_t)bh * a.n_int + iv;
  const int b0 = iv * a.S, b1 = min(b0 + a.S, a.nblk) - 1;
  const int ncand = a.cand_len[slot];
  if (ncand < 0) {                                     // too many candidates
    for (int blk = b1; blk >= b0; --blk) {
      full_select<kPwThreads>(a, blk, bh, s.ps);
      __syncthreads();
    }
    return;
  }
  const uint2* cp = a.cand + slot * kPsCap;
  for (int i = tid; i < ncand; i += kPwThreads) {
    const uint2 e = cp[i];
    s.w.key[i] = e.x;
    s.w.id[i] = (int32_t)e.y;
  }
  __syncthreads();
  LevelRanges lstart;
#pragma unroll
  for (int l = 0; l < 8; ++l) lstart.lo[l] = l < a.levels ? wave_lower_bound(s.w.id, ncand, a.soff[l], lane) : 0;
  const uint32_t lo = a.tau[slot], hi = a.tau_hi[slot];
  for (int blk = b1 - wid; blk >= b0; blk -= kPwWaves)
    wave_select(a, s, s.w.hist[wid], ncand, lstart, blk, bh, lo, hi, lane);
}

hipError_t launch_pyramid_select(const PyrSelectArgs& a, hipStream_t s) {
  if (!a.prefix) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pyr_prefix_kernel, dim3(a.B * a.H), dim3(1024), 0, s, a);
  if (a.n_int > 0) {
    if (a.S < 1 || !a.tau || !a.cand_len || !a.cand) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pyr_interval_kernel, dim3(a.n_int * a.B * a.H), dim3(kPiThreads), 0, s, a);
    hipLaunchKernelGGL(pyr_block_select_kernel, dim3(a.n_int * a.B * a.H), dim3(kPwThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(pyr_select_kernel, dim3(a.nblk, a.B * a.H), dim3(kPsThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace sa
