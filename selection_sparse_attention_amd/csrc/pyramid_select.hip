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
// One 256-thread workgroup per (block, sequence-head).  The K-th largest score
// key is resolved by radix levels of up to 12 bits over LDS histograms of the
// visible prefixes, with no sort; the digits start below the leading bits all
// keys of the head share (an AND/OR reduction over the head, one small launch
// first), so the buckets are well spread.  A final pass writes the kept flat
// ids in ascending order (strictly larger keys, then the first ties by flat
// id).
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
// flight.
__device__ void vis_hist(const float* sc, const VisRanges& v, uint32_t prefix, int pshift, int shift,
                         int bits, uint32_t* hist) {
  const uint32_t mask = (1u << bits) - 1u;
  for (int l = 0; l < v.nl; ++l) {
    const float* p = sc + v.off[l];
    const int cnt = v.cnt[l];
    for (int j0 = 0; j0 < cnt; j0 += kPsU * kPsThreads) {
      float x[kPsU];
#pragma unroll
      for (int u = 0; u < kPsU; ++u) {
        const int j = j0 + u * kPsThreads + threadIdx.x;
        x[u] = p[j < cnt ? j : cnt - 1];
      }
#pragma unroll
      for (int u = 0; u < kPsU; ++u) {
        const int j = j0 + u * kPsThreads + threadIdx.x;
        const uint32_t key = order_key(x[u]);
        if (j < cnt && (pshift >= 32 || (key >> pshift) == prefix))
          atomicAdd(&hist[(key >> shift) & mask], 1u);
      }
    }
  }
}

// Scan a histogram of NB buckets from the top for the bucket holding the
// `target`-th key; returns the bucket and adds the count above it to *above.
template <int NB>
__device__ int vis_find(const uint32_t* hist, int64_t target, int64_t* above, int64_t* s_scan,
                        int* s_b, int64_t* s_above) {
  constexpr int PER = NB / kPsThreads;
  const int tid = threadIdx.x;
  int64_t tc = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) tc += hist[NB - 1 - (PER * tid + k)];
  int64_t tot;
  const int64_t pre = block_exclusive_scan<int64_t, kPsThreads>(tc, s_scan, &tot);
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

__global__ __launch_bounds__(kPsThreads) void pyr_select_kernel(PyrSelectArgs a) {
  __shared__ uint32_t hist[4096];
  __shared__ int64_t s_scan[kPsThreads / 64];
  __shared__ uint32_t s_scan32[kPsThreads / 64];
  __shared__ int s_b;
  __shared__ int64_t s_above;
  // late blocks see the most entries: dispatch them first
  const int blk = a.nblk - 1 - (int)blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const VisRanges v = visible(a, blk);
  const float* sc = a.scores + (int64_t)bh * a.Nt;
  int32_t* out = a.blk_idx + ((int64_t)bh * a.nblk + blk) * a.K;
  const int64_t K = a.K;
  if (v.total <= K) {                      // every visible entry
    int64_t o = 0;
    for (int l = 0; l < v.nl; ++l) {
      for (int j = tid; j < v.cnt[l]; j += kPsThreads) out[o + j] = (int32_t)(v.off[l] + j);
      o += v.cnt[l];
    }
    if (tid == 0) a.blk_count[(int64_t)bh * a.nblk + blk] = (int32_t)v.total;
    return;
  }
  // The leading bits every key of the head shares carry no information: the
  // radix digits start below them (scores share sign and most exponent bits,
  // so a histogram of the top bits would pile everything into a few buckets).
  const uint2 pf = a.prefix[bh];
  const uint32_t diff = pf.x ^ pf.y;
  const int common = diff ? __clz(diff) : 32;
  int64_t above = 0;
  uint32_t cut = pf.x;                              // when every key is equal
  if (common < 32) {
    int pos = 32 - common;                          // bits still to resolve
    uint32_t prefix = pf.x >> pos;
    // digits of at most 12 bits
    while (pos > 0) {
      const int bits = pos < 12 ? pos : 12;
      const int shift = pos - bits;
      for (int i = tid; i < 4096; i += kPsThreads) hist[i] = 0;
      __syncthreads();
      vis_hist(sc, v, prefix, pos, shift, bits, hist);
      __syncthreads();
      const int bk = vis_find<4096>(hist, K, &above, s_scan, &s_b, &s_above);
      prefix = (prefix << bits) | (uint32_t)bk;
      pos = shift;
    }
    cut = prefix;
  }
  const uint32_t need = (uint32_t)(K - above);        // ties kept, lowest flat ids first

  // ascending flat ids: strict (key > cut) and the first `need` ties; thread
  // t takes kPsU consecutive entries of each chunk, loaded together
  uint32_t s_run = 0, t_run = 0;                      // totals of earlier chunks
  for (int l = 0; l < v.nl; ++l) {
    const float* p = sc + v.off[l];
    const int cnt = v.cnt[l];
    for (int j0 = 0; j0 < cnt; j0 += kPsU * kPsThreads) {
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
      const uint32_t ex_s = block_exclusive_scan<uint32_t, kPsThreads>(__popc(sf), s_scan32, &tot_s);
      const uint32_t ex_t = block_exclusive_scan<uint32_t, kPsThreads>(__popc(tf), s_scan32, &tot_t);
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

hipError_t launch_pyramid_select(const PyrSelectArgs& a, hipStream_t s) {
  if (!a.prefix) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pyr_prefix_kernel, dim3(a.B * a.H), dim3(1024), 0, s, a);
  dim3 grid(a.nblk, a.B * a.H);
  hipLaunchKernelGGL(pyr_select_kernel, grid, dim3(kPsThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
