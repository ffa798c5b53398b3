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
  int32_t tokens_per_wg; // key rows per workgroup
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
constexpr int kCap = 8192;         // candidate keys per row resolved in LDS
constexpr int kMaxSelW = 512;      // workgroups per selector row
// per-row control words of the selector workspace
constexpr int kCtlErr = 0;         // a wait timed out
constexpr int kCtlDepart = 1;      // workgroups that have left
constexpr int kCtlWords = 16;

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
  int32_t W;             // workgroups per row
  int32_t kv_div;        // rows per KV group of k_idx (G with per-head sets, else 1)
  int32_t spin_limit;    // polls per cross-workgroup wait (< 0: every wait fails)
  // fused append (bf16): project the rows' queries and token n - 1's index key
  // first, as the index build's append would (q_idx / k_idx are then written)
  int32_t append;
  int32_t d;             // head dim (64 or 128) of k_pre / q_pre
  const void* k_pre;     // [B,Hkv,n_cap,d]
  const void* q_pre;     // [B,Hq,d]
  const float* proj_q;   // [Hkv,16,d]
  const float* proj_k;   // [Hkv,16,d]
  float* q_idx_w;        // q_idx, written by the append
  void* k_idx_w;         // k_idx, row n - 1 written by the append
  // workspace; everything but `cand` is zero between calls
  uint32_t* hist_c;      // [rows, 3, 4096] counts of the three global digits
  double* hist_m;        // [rows, 3, 4096] masses of the three global digits
  uint32_t* ctl;         // [rows, kCtlWords]
  uint32_t* slot_a;      // [rows, kMaxSelW] last global digit each workgroup has merged
  uint64_t* slot_b;      // [rows, kMaxSelW] each workgroup's exchange counts (flagged)
  uint32_t* cand;        // [rows, cand_stride] candidate keys, one region of a tile per workgroup
  int64_t cand_stride;
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
  int32_t kv_div;               // selection rows per KV group (G with per-head sets, else 1)
  float* scratch;               // [rows, n_cs_cap] chunk scores
  GroupList groups;
  // chunked prefill: every query block of `chunk` queries routes (q is then
  // [B,Hq,n,d]); lists go to blk_idx [B,Hkv,nblk,K] / blk_count [B,Hkv,nblk]
  int32_t prefill;
  int32_t nblk, K;
  int32_t* blk_idx;
  int32_t* blk_count;
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
  // Hkv / G count selection groups: KV groups, or single query heads with
  // per-head sets (Hkv = Hq, G = 1); K/V rows belong to group index / kv_div
  int32_t B, Hq, Hkv, n, n_cap, G, sinks, window;
  int32_t kv_div;
  int32_t tps;            // tokens per split (fp32 path)
  int32_t max_splits;     // fp32 path: splits per group; bf16 path: work items
  float scale_log2;       // log2(e) / sqrt(d)
  uint64_t local_mask;    // bit g set: group g is local
  int32_t target_items;   // bf16 path: work items the visible tokens are spread over
  int32_t min_chunk;      // bf16 path: smallest item (list entries)
  int2* plan;             // bf16 path: per group (first item, item count) [B*Hkv]
  // monotone-gain early stop for the groups in `s2o` (bit g of s2o_mask
  // set): the split kernels run their first pass (the local rule) and the
  // combine caches each head's unnormalised state (m, l, acc[d]) in
  // s2o_state [B*Hkv*G, d+2] instead of writing outputs; the early-stop
  // kernel resumes from it over the candidates
  uint64_t s2o_mask;
  float s2o_tau;
  float* s2o_state;
  GroupList s2o;
  // per-head sets decoded per KV group: sel_idx / sel_count hold each
  // group's union of its heads' sets, an entry being (head mask << 24 |
  // position); head_count [B,Hq] are the heads' own counts (a negative one
  // poisons that head's output)
  int32_t head_masks;
  const int32_t* head_count;
};

// The union of the per-head sets of each selecting KV group.
struct HeadUnionArgs {
  const int32_t* sel_idx;     // [B,Hq,n_cap] each head's positions
  const int32_t* sel_count;   // [B,Hq]
  int32_t* union_idx;         // [B,Hkv,n_cap] (head mask << 24 | position), ascending
  int32_t* union_count;       // [B,Hkv]
  uint32_t* masks;            // [B,Hkv,mask_words] head bits, one byte per position
  int32_t* slice_count;       // [B,Hkv,n_slices] tagged positions per slice
  int32_t B, Hq, Hkv, G, n, n_cap, mask_words, n_slices;
  GroupList groups;           // the selecting KV groups
};

constexpr int kUnionMaxN = (1 << 24) - 1;  // positions an entry's 24 position bits hold
constexpr int kUnionSlice = 2048;          // positions per slice of the union

constexpr int kS2oMax = 8192;     // candidates per group the early-stop kernel stages

constexpr int kMaxPrefillHeads = 128;

struct PrefillArgs {
  const void* q; const void* k; const void* v;   // q [B,H,N,d]; k, v [B,Hkv,kv_stride,d]
  const void* pk; const void* pv;                // [B,H,Nc,d]
  const int32_t* blk_idx; const int32_t* blk_count;
  float* out;                                    // [B,H,N,d]
  float* lse;                                    // [B,H,N] or null: log of each row's softmax denominator
  int32_t B, H, N, Nc, nblk, K, q_block;
  float scale_log2;
  // head-split mode: the visible keys follow from each head's class - class
  // 0 dense causal, class 1 sinks + sliding window; query head h reads KV
  // head h / G
  int32_t Hkv, G, kv_stride, sinks, window;
  int32_t n_cls[2];                              // heads in each class
  int32_t units0;                                // workgroups of class 0
  uint8_t cls_heads[2][kMaxPrefillHeads];        // the heads of each class
  // coarse-query mode (lists, coarse != 0): the block's coarse query entries
  // of levels 1 .. levels-1 (rows of pq, level 1 first) attend in place of
  // its level-0 queries, each to the list and to the block's own entries of
  // its level up to itself; outputs to out_c [B,H,Nc,d]
  const void* pq;
  float* out_c;
  int32_t coarse, levels;
  int32_t c_off[8], c_span[8];                   // per level l >= 1: first coarse row, p^l
};

// Backward pass of the pyramid prefill: inputs as the forward's, the
// forward's outputs, the upstream gradient, the gradients, and workspace
// regions (per query delta = dO.O; per flat entry its last choosing block and
// the first row of its partial gradients; per head an error word; per-block
// partial gradients of the chosen entries; the coarse entries' sums).
struct BwdArgs {
  const void* q; const void* k; const void* v;   // [B,H,N,d] bf16
  const void* pk; const void* pv;                // [B,H,Nc,d] bf16
  const int32_t* blk_idx; const int32_t* blk_count;
  const float* out; const float* lse; const float* dout;
  float* dq; float* dk; float* dv;               // [B,H,N,d]
  float* delta;                                  // [B,H,N]
  int32_t* last;                                 // [B,H,E]
  int32_t* base;                                 // [B,H,E+1]
  uint32_t* err;                                 // [B,H]
  uint16_t* part_k; uint16_t* part_v;            // [B,H,R,d] bf16
  float* coarse_k; float* coarse_v;              // [B,H,Nc,d]
  int64_t R;                                     // partial rows per head (the last is a spare)
  int32_t B, H, N, Nc, E, nblk, K, q_block, levels;
  int32_t off[8], span[8], cnt[8];               // per level: flat offset, rows covered, entries
  float scale, scale_log2;
};

// Tiered K/V of the routed decode: the routed lists are served from a cold
// host store through warm device slots (one routing group each, LRU) and
// rewritten as rows of the device tier (hot rows, then the warm slots).
struct TierArgs {
  const int32_t* sel_idx;        // [B,Hkv,n_cap] routed positions
  int32_t* rows;                 // [B,Hkv,dev_rows] the lists as rows of the device tier
  const int32_t* sel_count;      // [B,Hkv]
  const char* cold_k; const char* cold_v;   // device-visible host memory [B,Hkv,n_cap,row_bytes]
  char* dev_k; char* dev_v;      // [B,Hkv,dev_rows,row_bytes]
  int32_t* slot_group;           // [B,Hkv,warm_slots]
  int32_t* slot_stamp;           // [B,Hkv,warm_slots]
  int32_t* stats;                // [B,Hkv,2] or null
  int32_t B, Hkv, n, n_cap, row_bytes, chunk, group, sink_chunks, local_chunks;
  int32_t warm_slots, dev_rows, step;
  GroupList groups;              // the routed KV groups
};

constexpr int kTierListMax = 8192;       // longest routed list a fetch stages
constexpr int kTierSlotsMax = 4096;      // warm slots per (sequence, KV group)
constexpr int kTierNeedMax = 256;        // routed groups per list

// ---------------------------------------------------------------- launchers
hipError_t launch_index_lowrank(const IndexLowrankArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_summary(const SummaryArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_pyramid(const PyramidArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_select_lowrank(const SelectArgs& a, int dtype, int per, hipStream_t s);
hipError_t launch_route(const RouteArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_pyramid_select(const PyrSelectArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, hipStream_t s);
hipError_t launch_decode_mfma(const DecodeArgs& a, int d, hipStream_t s);
hipError_t launch_decode_s2o(const DecodeArgs& a, int d, hipStream_t s);
hipError_t launch_head_union(const HeadUnionArgs& a, hipStream_t s);
hipError_t launch_tier_fetch(const TierArgs& a, hipStream_t s);
hipError_t launch_select_order(const SelectArgs& a, int dtype, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int d, hipStream_t s);
hipError_t launch_prefill_heads(const PrefillArgs& a, int d, hipStream_t s);
hipError_t launch_prefill_backward(const BwdArgs& a, int d, hipStream_t s);

}  // namespace sa
