// Tiered K/V storage of the routed decode ("Atencao Global Hierarquica
// (HGA)" summary, Memory architecture: the whole K/V history in host RAM
// (cold), a bounded LRU cache of recently routed blocks in device memory
// (warm), summaries and the always-visible windows in device memory (hot);
// Core mechanism item 4: the router brings the routed groups' original
// token-level K/V rows from host RAM into device memory).
//
// One 256-thread workgroup per (routed KV group, sequence), run after the
// routing and before the decode:
//   1. the routed list (ascending positions) is staged in LDS; the distinct
//      routing groups of its routed part (positions between the sink chunks
//      and the local window) are compacted in order;
//   2. the warm slots' (group, last use) tables are staged; a slot holding a
//      needed group is a hit and takes this step's stamp;
//   3. the other slots are ranked by (in use, last use, slot index) with a
//      bitonic sort of 64-bit keys: the missing groups, in ascending order,
//      take the first of them (empty slots, then least recently used);
//   4. the missing groups' K and V rows are copied from the cold store (host
//      memory the device reads directly, over the host link) into their
//      slots, 16 bytes per thread per access;
//   5. the list is written out as rows of the device tier: a sink position
//      is its own row, a local-window or current-chunk position p the ring
//      row sink_rows + p mod ring, a routed position its slot's row.
// Every decision follows a fixed order, so the tables evolve the same way in
// every run.  The decode then runs over the device tier unchanged.
#include "args.hpp"
#include "common.hpp"

namespace sa {

constexpr int kTierThreads = 256;

__global__ __launch_bounds__(kTierThreads) void tier_fetch_kernel(TierArgs a) {
  __shared__ int32_t s_list[kTierListMax];
  __shared__ int32_t s_need[kTierNeedMax];
  __shared__ int32_t s_place[kTierNeedMax];     // slot of each needed group
  __shared__ int32_t s_hit[kTierNeedMax];       // 1: already warm
  __shared__ uint64_t s_key[kTierSlotsMax];     // rank of the free slots
  __shared__ int32_t s_scan[kTierThreads / 64];
  __shared__ int32_t s_nmiss;
  const int g = a.groups.ids[blockIdx.x], b = blockIdx.y, tid = threadIdx.x;
  const int64_t bg = (int64_t)b * a.Hkv + g;
  const int cnt = min(a.sel_count[bg], kTierListMax);
  if (cnt < 0) return;                          // a failed routing: the decode poisons it
  const int32_t* list = a.sel_idx + bg * a.n_cap;
  int32_t* rows = a.rows + bg * a.dev_rows;
  const int C = a.chunk, grp = a.group;
  const int sink_rows = a.sink_chunks * C;
  const int ring = (a.local_chunks + 1) * C;
  const int hot_rows = sink_rows + ring;
  const int kappa = (a.n - 1) / C;
  const int win_lo = (kappa - a.local_chunks) * C;      // first position of the local window
  auto routed = [&](int p) __attribute__((always_inline)) { return p >= sink_rows && p < win_lo; };

  // ---- 1. the list and its distinct routed groups, in order
  for (int i = tid; i < cnt; i += kTierThreads) s_list[i] = list[i];
  __syncthreads();
  const int per = (cnt + kTierThreads - 1) / kTierThreads;
  const int i0 = min(cnt, tid * per), i1 = min(cnt, i0 + per);
  int firsts = 0;
  for (int i = i0; i < i1; ++i) {
    const int p = s_list[i];
    if (routed(p) && (i == 0 || !routed(s_list[i - 1]) || s_list[i - 1] / grp != p / grp)) ++firsts;
  }
  int nneed;
  int o = block_exclusive_scan<int32_t, kTierThreads>(firsts, s_scan, &nneed);
  for (int i = i0; i < i1; ++i) {
    const int p = s_list[i];
    if (routed(p) && (i == 0 || !routed(s_list[i - 1]) || s_list[i - 1] / grp != p / grp)) {
      if (o < kTierNeedMax) s_need[o] = p / grp;
      ++o;
    }
  }
  nneed = min(nneed, kTierNeedMax);
  for (int k = tid; k < nneed; k += kTierThreads) { s_hit[k] = 0; s_place[k] = -1; }
  __syncthreads();

  // ---- 2. hits: a slot that holds a needed group (binary search in s_need)
  int32_t* sg = a.slot_group + bg * a.warm_slots;
  int32_t* ss = a.slot_stamp + bg * a.warm_slots;
  const int S = a.warm_slots;
  int P = 2;
  while (P < S) P <<= 1;
  for (int sl = tid; sl < P; sl += kTierThreads) {
    uint64_t key = ~0ull;                       // not a candidate
    if (sl < S) {
      const int gs = sg[sl];
      int lo = 0, hi = nneed;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_need[mid] < gs) lo = mid + 1; else hi = mid;
      }
      if (gs >= 0 && lo < nneed && s_need[lo] == gs) {
        s_hit[lo] = 1;
        s_place[lo] = sl;
      } else {
        // free slots first, then by last use, then by index
        key = ((uint64_t)(gs >= 0) << 62) | ((uint64_t)(uint32_t)ss[sl] << 20) | (uint64_t)sl;
      }
    }
    s_key[sl] = key;
  }
  __syncthreads();

  // ---- 3. rank the candidate slots (ascending keys), when a group misses
  int nmiss_local = 0;
  for (int k = tid; k < nneed; k += kTierThreads) nmiss_local += !s_hit[k];
  const bool any_miss = __syncthreads_or(nmiss_local) != 0;
  for (int k = 2; k <= P && any_miss; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kTierThreads) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = s_key[i], y = s_key[ixj];
          if ((x > y) == ((i & k) == 0)) { s_key[i] = y; s_key[ixj] = x; }
        }
      }
      __syncthreads();
    }
  }
  // the missing groups take the first candidates in order
  if (tid < 64 && !any_miss) {
    if (tid == 0) s_nmiss = 0;
  } else if (tid < 64) {
    int base = 0;
    for (int k0 = 0; k0 < nneed; k0 += 64) {
      const int k = k0 + tid;
      const bool miss = k < nneed && !s_hit[k];
      const uint64_t bal = __ballot(miss);
      const int rank = base + __popcll(bal & ((tid == 0) ? 0ull : (~0ull >> (64 - tid))));
      if (miss) {
        const uint64_t key = (rank < P) ? s_key[rank] : ~0ull;
        const int sl = (int)(key & 0xFFFFFu);
        s_place[k] = (key == ~0ull || sl >= S) ? -1 : sl;
      }
      base += __popcll(bal);
    }
    if (tid == 0) s_nmiss = base;
  }
  __syncthreads();

  // ---- 4. tables, and the missing groups' rows from the cold store
  for (int k = tid; k < nneed; k += kTierThreads) {
    const int sl = s_place[k];
    if (sl < 0) continue;                       // more groups than slots: rejected on the host
    if (!s_hit[k]) sg[sl] = s_need[k];
    ss[sl] = a.step;
  }
  const int units = a.row_bytes / 16;           // 16-byte units per row
  const int per_group = grp * units;
  const int64_t cold0 = bg * a.n_cap;
  const int64_t dev0 = bg * a.dev_rows;
  for (int k = 0; k < nneed; ++k) {
    if (s_hit[k] || s_place[k] < 0) continue;
    const int64_t src_row = cold0 + (int64_t)s_need[k] * grp;
    const int64_t dst_row = dev0 + hot_rows + (int64_t)s_place[k] * grp;
    for (int u = tid; u < per_group; u += kTierThreads) {
      const int r = u / units, c = u - r * units;
      const int64_t so = (src_row + r) * a.row_bytes + 16 * c;
      const int64_t dso = (dst_row + r) * a.row_bytes + 16 * c;
      const uint4 kv = *reinterpret_cast<const uint4*>(a.cold_k + so);
      const uint4 vv = *reinterpret_cast<const uint4*>(a.cold_v + so);
      *reinterpret_cast<uint4*>(a.dev_k + dso) = kv;
      *reinterpret_cast<uint4*>(a.dev_v + dso) = vv;
    }
  }

  // ---- 5. the list as rows of the device tier (at most dev_rows entries:
  //      the hot rows plus the routed groups, which fit in the slots)
  for (int i = tid; i < min(cnt, a.dev_rows); i += kTierThreads) {
    const int p = s_list[i];
    int row;
    if (p < sink_rows) {
      row = p;
    } else if (p >= win_lo) {
      row = sink_rows + p % ring;
    } else {
      const int gid = p / grp;
      int lo = 0, hi = nneed;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_need[mid] < gid) lo = mid + 1; else hi = mid;
      }
      const int sl = (lo < nneed && s_need[lo] == gid) ? s_place[lo] : -1;
      row = (sl >= 0) ? hot_rows + sl * grp + p % grp : -1;   // -1: never attended
    }
    rows[i] = row;
  }
  if (a.stats && tid == 0) {
    a.stats[2 * bg] = nneed - s_nmiss;
    a.stats[2 * bg + 1] = s_nmiss;
  }
}

hipError_t launch_tier_fetch(const TierArgs& a, hipStream_t s) {
  if (a.warm_slots < 1 || a.warm_slots > kTierSlotsMax || a.group < 1 || a.chunk % a.group) return hipErrorInvalidValue;
  if (a.row_bytes % 16 || a.dev_rows != (a.sink_chunks + a.local_chunks + 1) * a.chunk + a.warm_slots * a.group)
    return hipErrorInvalidValue;
  if (a.groups.n == 0 || a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(tier_fetch_kernel, dim3(a.groups.n, a.B), dim3(kTierThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace sa
