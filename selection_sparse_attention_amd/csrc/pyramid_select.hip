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
// key is resolved by three radix levels (12 + 12 + 8 bits) of LDS histograms
// over the visible prefixes, with no sort; a final pass writes the kept flat
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

// Histogram of the visible keys whose top bits match `prefix` (pshift bits
// above the bucket field), bucket = (key >> shift) & (NB - 1).
template <int NB>
__device__ void vis_hist(const float* sc, const VisRanges& v, uint32_t prefix, int pshift,
                         int shift, uint32_t* hist) {
  for (int l = 0; l < v.nl; ++l) {
    const float* p = sc + v.off[l];
    for (int j = threadIdx.x; j < v.cnt[l]; j += kPsThreads) {
      const uint32_t key = order_key(p[j]);
      if (pshift >= 32 || (key >> pshift) == prefix) atomicAdd(&hist[(key >> shift) & (NB - 1)], 1u);
    }
  }
}

// Scan a histogram from the top for the bucket holding the `target`-th key;
// returns the bucket and adds the count above it to *above.
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
  const int blk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
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
  // level 1: bits 31..20
  int64_t above = 0;
  for (int i = tid; i < 4096; i += kPsThreads) hist[i] = 0;
  __syncthreads();
  vis_hist<4096>(sc, v, 0, 32, 20, hist);
  __syncthreads();
  const int b1 = vis_find<4096>(hist, K, &above, s_scan, &s_b, &s_above);
  // level 2: bits 19..8 inside b1
  for (int i = tid; i < 4096; i += kPsThreads) hist[i] = 0;
  __syncthreads();
  vis_hist<4096>(sc, v, (uint32_t)b1, 20, 8, hist);
  __syncthreads();
  const int b2 = vis_find<4096>(hist, K, &above, s_scan, &s_b, &s_above);
  // level 3: bits 7..0
  for (int i = tid; i < 256; i += kPsThreads) hist[i] = 0;
  __syncthreads();
  const uint32_t p2 = ((uint32_t)b1 << 12) | (uint32_t)b2;
  vis_hist<256>(sc, v, p2, 8, 0, hist);
  __syncthreads();
  const int b3 = vis_find<256>(hist, K, &above, s_scan, &s_b, &s_above);
  const uint32_t cut = (p2 << 8) | (uint32_t)b3;
  const uint32_t need = (uint32_t)(K - above);        // ties kept, lowest flat ids first

  // ascending flat ids: strict (key > cut) and the first `need` ties
  uint32_t s_run = 0, t_run = 0;                      // totals of earlier chunks
  for (int l = 0; l < v.nl; ++l) {
    const float* p = sc + v.off[l];
    for (int j0 = 0; j0 < v.cnt[l]; j0 += 4 * kPsThreads) {
      uint32_t sf = 0, tf = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * tid + i;
        if (j < v.cnt[l]) {
          const uint32_t key = order_key(p[j]);
          if (key > cut) sf |= 1u << i;
          else if (key == cut) tf |= 1u << i;
        }
      }
      uint32_t tot_s, tot_t;
      const uint32_t ex_s = block_exclusive_scan<uint32_t, kPsThreads>(__popc(sf), s_scan32, &tot_s);
      const uint32_t ex_t = block_exclusive_scan<uint32_t, kPsThreads>(__popc(tf), s_scan32, &tot_t);
      uint32_t sb = s_run + ex_s, tb = t_run + ex_t;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * tid + i;
        if (sf & (1u << i)) {
          out[sb + (tb < need ? tb : need)] = (int32_t)(v.off[l] + j);
          ++sb;
        } else if (tf & (1u << i)) {
          if (tb < need) out[sb + tb] = (int32_t)(v.off[l] + j);
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
  dim3 grid(a.nblk, a.B * a.H);
  hipLaunchKernelGGL(pyr_select_kernel, grid, dim3(kPsThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
