// Launch argument structs passed by value from the host layer to kernels,
// and the host-side launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kMaxGroups = 64;   // KV heads supported per call
constexpr int kMaxTps = 1024;    // decode: most list entries per split

// The KV groups a kernel works on (retrieval, routed or local groups).
struct GroupList {
  int32_t n;
  int32_t ids[kMaxGroups];
};

// ---------------------------------------------------------------- index
struct IndexLowrankArgs {
  const void* k_pre;     // [B,Hkv,n_cap,d]
  const void* q_pre;     // [B,Hq,d] or nullptr
  const float* proj_q;   // [Hkv,16,d]
  const float* proj_k;   // [Hkv,16,d]
  void* k_idx;           // [B,Hkv,n_cap,16]
  float* q_idx;          // [B,Hq,16]
  int32_t B, Hq, Hkv, n_cap, G, t0, t1;
  GroupList groups;
};

struct SummaryArgs {
  const void* k_pre;     // [B,Hkv,n_cap,d]
  void* chunk_sum;       // [B,Hkv,n_cap/chunk,d]
  void* group_sum;       // [B,Hkv,n_cap/group,d]
  int32_t B, Hkv, n_cap, chunk, group;
  int32_t c0, c1;        // chunk range [c0, c1) to build
  int32_t g0, g1;        // group range [g0, g1) to build
  double rope_base;
  GroupList groups;
};

struct PyramidArgs {
  const void* q; const void* k; const void* v;     // [B,H,N,d]
  void* pq; void* pk; void* pv;                    // [B,H,Nc,d]
  float* scores;                                   // [B,H,Nt]
  int32_t B, H, N, levels, factor, Nc, Nt;
  int32_t top_span;                                // p^(L-1)
  int64_t coff[8];                                 // row of level l's first entry in pq/pk/pv
  int64_t soff[8];                                 // flat id of level l's first entry
};

// ---------------------------------------------------------------- select
// Per-row (sequence, retrieval group) state of the radix selector.
struct RowState {
  double R;             // reference logit: masses are exp(l - R)
  double target_mass;   // p * total mass
  double mass_above;    // mass of tokens above the current key prefix
  int64_t count_above;  // tokens above the current key prefix
  int32_t target_count; // min_tokens or k
  uint32_t prefix;      // key bits fixed so far
  int32_t crit;         // bit0: mass criterion live, bit1: count criterion live
  int32_t all;          // 1: every token is selected
  uint32_t cut_key;     // final key of the last selected token
  int32_t need;         // tokens taken among those whose key == cut_key
  int32_t m;            // selected count
  int32_t err;
};

struct SelectArgs {
  const float* q_idx;    // [B,Hq,16]
  const void* k_idx;     // [B,Hkv,n_cap,16]
  int32_t* sel_idx;      // [B,Hkv,n_cap]
  int32_t* sel_count;    // [B,Hkv]
  int32_t B, Hq, Hkv, n, n_cap, G;
  int32_t use_mass;      // 1 = top-p, 0 = top-k
  int32_t select_all;    // every token is kept (no ranking needed)
  double top_p;
  int32_t target_count;  // top-k: k ; top-p: min_tokens (0 = none)
  int32_t tiles;         // tiles per row
  int64_t row_stride;    // logits stride per row (tiles * tile)
  // workspace
  float* logits;         // [rows, row_stride]
  uint32_t* cnt1; double* mass1;   // [rows, 4096]: level-1 histogram, zero between calls
  uint32_t* maxkey;      // [rows]: largest order key of the row's logits, zero between calls
  RowState* state;       // [rows]: the cut found by the row kernel
  uint64_t* lookback;    // [rows, tiles]: compaction prefix flags
  GroupList groups;
};

struct RouteArgs {
  const void* q;          // [B,Hq,d] post-RoPE
  const void* chunk_sum;  // [B,Hkv,n_cap/chunk,d]
  const void* group_sum;  // [B,Hkv,n_cap/group,d]
  int32_t* sel_idx; int32_t* sel_count;
  int32_t B, Hq, Hkv, n, n_cap, G, chunk, group, top_chunks, top_groups,
      sink_chunks, local_chunks;
  int32_t n_cs_cap, n_gs_cap;   // rows per (b,g) in chunk_sum / group_sum
  float* scratch;               // [rows, n_cs_cap] chunk scores
  GroupList groups;
};

struct PyrSelectArgs {
  const float* scores;   // [B,H,Nt]
  int32_t* blk_idx;      // [B,H,nblk,K]
  int32_t* blk_count;    // [B,H,nblk]
  int32_t B, H, N, levels, factor, q_block, K, nblk, Nt;
  int32_t len[8];        // entries of each level
  int64_t soff[8];       // flat id of each level's first entry
  uint2* prefix;         // workspace [B*H]: (AND, OR) of the head's score keys
  // intervals of S consecutive blocks (n_int per head; 0 = not used)
  int32_t S, n_int;
  uint32_t* tau;         // [B*H, n_int]: cut key of the interval's first block
  uint32_t* tau_hi;      // [B*H, n_int]: cut key of the interval's last block
  int32_t* cand_len;     // [B*H, n_int]: candidates kept (-1: more than kPsCap)
  uint2* cand;           // [B*H, n_int, kPsCap]: (key, flat id), ascending flat id
};

constexpr int kPsCap = 7680;   // candidate slots per interval (and LDS entries per block)

// ---------------------------------------------------------------- attention
struct DecodeArgs {
  const void* q;          // [B,Hq,d]
  const void* k;          // [B,Hkv,n_cap,d]
  const void* v;
  const int32_t* sel_idx; // [B,Hkv,n_cap]
  const int32_t* sel_count;
  float* out;             // [B,Hq,d]
  float* partial;         // [B,Hq,max_splits,d+2]
  int32_t B, Hq, Hkv, n, n_cap, G, sinks, window;
  int32_t tps;            // tokens per split (fp32 path)
  int32_t max_splits;     // fp32 path: splits per group; bf16 path: work items
  float scale_log2;       // log2(e) / sqrt(d)
  uint64_t local_mask;    // bit g set: group g is local
  int32_t target_items;   // bf16 path: work items the visible tokens are spread over
  int32_t min_chunk;      // bf16 path: smallest item (list entries)
  int2* plan;             // bf16 path: per group (first item, item count) [B*Hkv]
};

struct PrefillArgs {
  const void* q; const void* k; const void* v;   // [B,H,N,d]
  const void* pk; const void* pv;                // [B,H,Nc,d]
  const int32_t* blk_idx; const int32_t* blk_count;
  float* out;                                    // [B,H,N,d]
  int32_t B, H, N, Nc, nblk, K, q_block;
  float scale_log2;
};

// ---------------------------------------------------------------- launchers
hipError_t launch_index_lowrank(const IndexLowrankArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_summary(const SummaryArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_pyramid(const PyramidArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_select_lowrank(const SelectArgs& a, int dtype, hipStream_t s);
hipError_t launch_route(const RouteArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_pyramid_select(const PyrSelectArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int d, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int d, hipStream_t s);

}  // namespace sa
