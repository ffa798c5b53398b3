/*
 * sparse_attn.h - C ABI of a selection-based sparse attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (summarised on five public web pages, cited below by page title
 * and section) scores the history cheaply, selects a subset per KV group or
 * per query block, and runs exact softmax attention over only the selected
 * keys/values:
 *
 *  - "Full Attention Strikes Back" summary (RTPurbo), Methodology items 1-3, 5:
 *    retrieval heads select tokens with a 16-dim pre-RoPE low-rank index and a
 *    dynamic top-p (or static top-k) selector; local heads keep attention
 *    sinks plus a sliding window.
 *  - "Atencao Global Hierarquica (HGA)" summary, Core mechanism items 1-4:
 *    64-token chunks split into groups, two-level routing over RoPE-aware
 *    chunk/group key summaries, always-visible sink/local/current chunks,
 *    exact token attention over the routed set.
 *  - "Lighthouse Attention" summary, Methodology 2A-2C: symmetric mean
 *    pyramid over Q/K/V, l2-norm scores with max inheritance, joint top-K
 *    across levels per query block, dense attention on the gathered entries,
 *    outputs written back to their positions.
 *  - "Autonomia de Cabecas (AoH)" summary, Methodology item 4: GQA heads are
 *    aggregated to their group by the mean; sinks + recent window.
 *
 * Conventions common to every entry point
 *  - Ownership: the caller allocates every device buffer and the workspace;
 *    the library never allocates or frees memory, keeps no pointer after a
 *    call returns and holds no mutable global state.  Calls on different
 *    streams with disjoint output and workspace buffers may run concurrently.
 *  - Streams: all device work is enqueued on `hip_stream` (a hipStream_t; NULL
 *    means the default stream).  No call synchronises or copies device memory
 *    to the host; data-dependent sizes (selected counts) stay on the device.
 *  - Layouts: dense, row-major, in the order written for each buffer.  Token
 *    stride of every per-token buffer is `n_cap` (>= n_ctx).  Element type of
 *    queries, keys, values, index keys, summaries and pyramid levels is
 *    `params->dtype`; projectors, index queries, scores and outputs are fp32;
 *    lists are int32.  All device pointers must be 16-byte aligned; the
 *    workspace 256-byte aligned.
 *  - Workspace: pass workspace == NULL to read the required size into
 *    *workspace_bytes (nothing is validated against device data and nothing is
 *    launched); otherwise *workspace_bytes must hold the size of the buffer
 *    given, and a smaller value returns SA_ERR_WORKSPACE.  A workspace must be
 *    zero-filled before its first use and left untouched by the caller between
 *    calls: it carries histograms and counters that every completed call
 *    returns to zero (after SA_ERR_HIP, zero-fill it again).  Their offsets
 *    depend on batch, the head counts and the head kinds (not on n_ctx): after
 *    a call with different values of those, zero-fill it again.  Calls that
 *    may run concurrently need distinct workspaces.
 *  - Errors: arguments are validated on the host before anything is launched;
 *    an invalid argument launches nothing.  A failed launch returns SA_ERR_HIP
 *    (work enqueued before it may still run).  Faults inside kernels surface at
 *    the caller's next synchronisation.
 *  - Query position: decode queries sit at t = n_ctx - 1 and the cache holds
 *    keys 0 .. n_ctx - 1 (the current token included).
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSE_ATTN_VERSION 1

typedef enum {
  SA_OK = 0,
  SA_ERR_INVALID_ARG = -1,  /* a shape, parameter, label or pointer is invalid */
  SA_ERR_UNSUPPORTED = -2,  /* valid but not implemented (e.g. head_dim 96)   */
  SA_ERR_WORKSPACE = -3,    /* workspace smaller than required                */
  SA_ERR_CAPACITY = -4,     /* n_cap too small for the lists to be written    */
  SA_ERR_HIP = -5           /* a HIP launch returned an error                 */
} sa_status;

typedef enum { SA_BF16 = 0, SA_FP32 = 1 } sa_dtype;

/* Per-query-head label.  Labels must be equal inside a GQA group. */
typedef enum {
  SA_HEAD_LOCAL = 0,      /* sinks + sliding window                        */
  SA_HEAD_RETRIEVAL = 1,  /* low-rank index + top-p / top-k                */
  SA_HEAD_ROUTED = 2      /* chunk -> group routing over key summaries     */
} sa_head_kind;

typedef enum {
  SA_IDX_LOWRANK = 0,        /* k_idx rows (+ q_idx) for retrieval groups  */
  SA_IDX_CHUNK_SUMMARY = 1,  /* chunk and group key summaries              */
  SA_IDX_PYRAMID = 2         /* coarse Q/K/V levels and entry scores       */
} sa_index_mode;

typedef enum {
  SA_SEL_TOPP = 0,          /* retrieval groups: top-p mass, min_tokens floor */
  SA_SEL_TOPK = 1,          /* retrieval groups: fixed top_k                  */
  SA_SEL_ROUTE2 = 2,        /* routed groups: chunk then group routing        */
  SA_SEL_PYRAMID_TOPK = 3   /* per query block: joint top-K over levels       */
} sa_select_mode;

/* Host struct, read only during the call. */
typedef struct sa_params {
  int32_t batch;        /* B                                                   */
  int32_t n_q_heads;    /* Hq                                                  */
  int32_t n_kv_heads;   /* Hkv; Hq % Hkv == 0 (GQA group size G = Hq / Hkv)    */
  int32_t head_dim;     /* d: 64 or 128                                        */
  int32_t n_ctx;        /* n: keys in the cache / tokens in the prefill        */
  int32_t n_cap;        /* token stride of per-token buffers, >= n_ctx         */
  int32_t dtype;        /* sa_dtype                                            */
  const int8_t* head_kind; /* host array [Hq] of sa_head_kind                  */
  float rope_base;      /* RoPE base for the chunk summaries                   */
  int32_t r;            /* low-rank index width, must be 16                    */
  float top_p;          /* SA_SEL_TOPP: 0 < p <= 1 (p >= 1 keeps every token)  */
  int32_t top_k;        /* SA_SEL_TOPK: k >= 1                                 */
  int32_t min_tokens;   /* SA_SEL_TOPP: lower bound on the selected count      */
  int32_t sinks;        /* local heads: first `sinks` tokens                   */
  int32_t window;       /* local heads: last `window` tokens incl. the query   */
  int32_t chunk;        /* routing: chunk size C                               */
  int32_t group;        /* routing: group size; chunk % group == 0             */
  int32_t top_chunks;   /* routing: chunks kept at level 1                     */
  int32_t top_groups;   /* routing: groups kept per chunk at level 2           */
  int32_t sink_chunks;  /* routing: always-visible leading chunks              */
  int32_t local_chunks; /* routing: always-visible chunks before the current   */
  int32_t levels;       /* pyramid: L >= 1                                     */
  int32_t factor;       /* pyramid: p >= 2                                     */
  int32_t q_block;      /* pyramid: queries per block; % p^(L-1) == 0          */
  int32_t block_top_k;  /* pyramid: K entries per block                        */
} sa_params;

/* Device pointers owned by the caller; NULL where a call does not use them. */
typedef struct sa_buffers {
  const void* q_pre;    /* [B,Hq,d]           pre-RoPE decode query            */
  const void* k_pre;    /* [B,Hkv,n_cap,d]    pre-RoPE keys                    */
  const void* q;        /* [B,Hq,d] post-RoPE decode query | [B,H,N,d] prefill Q */
  const void* k_cache;  /* [B,Hkv,n_cap,d]    post-RoPE keys | prefill level-0 K */
  const void* v_cache;  /* [B,Hkv,n_cap,d]    values | prefill level-0 V         */
  const float* proj_q;  /* [Hkv,r,d] fp32     index projector, query side      */
  const float* proj_k;  /* [Hkv,r,d] fp32     index projector, key side        */
  float* q_idx;         /* [B,Hq,r] fp32      index queries                    */
  void* k_idx;          /* [B,Hkv,n_cap,r]    index keys                       */
  void* chunk_sum;      /* [B,Hkv,n_cap/chunk,d] chunk key summaries           */
  void* group_sum;      /* [B,Hkv,n_cap/group,d] group key summaries           */
  void* pyr_q;          /* [B,H,Nc,d] coarse levels 1..L-1 back to back,       */
  void* pyr_k;          /*            Nc = sum_{l>=1} N/p^l, level 1 first     */
  void* pyr_v;
  float* pyr_scores;    /* [B,H,Nt] fp32, Nt = sum_{l>=0} N/p^l, level 0 first */
  int32_t* sel_idx;     /* [B,Hkv,n_cap] selected positions, ascending         */
  int32_t* sel_count;   /* [B,Hkv] number of valid entries in sel_idx          */
  int32_t* blk_idx;     /* [B,H,ceil(N/q_block),K] flat entry ids per block    */
  int32_t* blk_count;   /* [B,H,ceil(N/q_block)]                               */
  float* out;           /* [B,Hq,d] decode | [B,H,N,d] prefill, fp32           */
} sa_buffers;

/*
 * sparse_attn_index_build - build (or extend) the cheap scorer's index.
 *
 * SA_IDX_LOWRANK ("Full Attention Strikes Back" summary, Methodology item 2):
 *   k_idx[b,g,j,:] = P_k[g] k_pre[b,g,j,:] for j in [t_begin, t_end) and every
 *   KV group whose heads are retrieval heads (fp32 accumulation, rounded once
 *   to dtype); q_idx[b,h,:] = P_q[g(h)] q_pre[b,h,:] (fp32) for every retrieval
 *   head when q_pre is not NULL.  Reads k_pre, proj_k, (q_pre, proj_q).
 * SA_IDX_CHUNK_SUMMARY (HGA summary, Core mechanism item 3): for every chunk
 *   (and every group) whose last token lies in [t_begin, t_end), writes the
 *   mixed RoPE summary of its pre-RoPE keys: pair i (dims i, i + d/2) is high
 *   frequency iff theta_i * (span - 1) > 1 rad, theta_i = base^(-2i/d); high
 *   pairs are rotated per token then averaged, low pairs are averaged then
 *   rotated at the span's mean position.  Angles are formed in fp64.  Every
 *   KV group whose heads are routed.  Reads k_pre; writes chunk_sum, group_sum.
 * SA_IDX_PYRAMID (Lighthouse summary, 2A-2B): builds levels 1..L-1 of Q, K and
 *   V (each entry the mean of its p^l level-0 rows, rounded once to dtype)
 *   and the entry scores: |q_i|^2 + |k_i|^2 at level 0, the max over children
 *   above.  Requires t_begin == 0 and t_end == n_ctx; n_ctx % p^(L-1) == 0;
 *   n_q_heads == n_kv_heads.  Reads q, k_cache, v_cache; writes pyr_*.
 *
 * No workspace.  Returns SA_ERR_INVALID_ARG for an empty or out-of-range
 * [t_begin, t_end) and SA_ERR_UNSUPPORTED for r != 16 or d not in {64, 128}.
 */
int32_t sparse_attn_index_build(const sa_params* params, const sa_buffers* bufs,
                                int32_t mode, int32_t t_begin, int32_t t_end,
                                void* hip_stream);

/*
 * sparse_attn_select - pick the token set of every selecting KV group, or the
 * entry set of every query block.
 *
 * SA_SEL_TOPP / SA_SEL_TOPK ("Full Attention Strikes Back" summary,
 *   Methodology items 2-3 and 5; AoH summary, item 4): for each retrieval
 *   group, qbar = mean of its heads' q_idx; logit l_j = qbar . k_idx_j / 4
 *   (= 1/sqrt(r)); tokens are ranked by (l desc, j asc).  TOPP keeps the
 *   shortest prefix whose softmax mass reaches top_p (all tokens when
 *   top_p >= 1), raised to min_tokens and capped at n_ctx; TOPK keeps
 *   min(top_k, n_ctx).  The cut is found by radix histograms over
 *   order-preserving logit keys with masses accumulated in fp64 (no sort).
 *   Writes sel_idx (ascending) and sel_count for those groups.
 * SA_SEL_ROUTE2 (HGA summary, Core mechanism item 2): for each routed group,
 *   qbar = mean of its post-RoPE queries q; with t = n_ctx - 1 and
 *   kappa = t / chunk, the chunks in [sink_chunks, kappa - local_chunks) are
 *   ranked by qbar . chunk_sum (ties to the lower chunk), the top top_chunks
 *   kept, and in each the top top_groups groups by qbar . group_sum.  The list
 *   is the union of sink chunks, local chunks, tokens kappa*chunk .. t, and
 *   the routed groups, ascending.  Needs n_cap >= the list length;
 *   top_chunks <= 64 and chunk / group <= 64 (SA_ERR_UNSUPPORTED otherwise).
 * SA_SEL_PYRAMID_TOPK (Lighthouse summary, 2B-2C): for every block of q_block
 *   queries, among entries (l, j) with (j + 1) p^l <= q_block * block, keeps
 *   the block_top_k largest pyr_scores (ties: lower level, then lower j) as
 *   flat ids off_l + j (off_0 = 0, off_l = sum_{m<l} N/p^m) in blk_idx, in
 *   no particular order, with the count in blk_count.
 *
 * Needs a workspace (size query as described above).
 */
int32_t sparse_attn_select(const sa_params* params, const sa_buffers* bufs,
                           int32_t mode, void* workspace, size_t* workspace_bytes,
                           void* hip_stream);

/*
 * sparse_attn_decode - exact softmax attention of each decode query head over
 * its group's visible set (HGA summary, Core mechanism item 4; "Full
 * Attention Strikes Back" summary, Methodology items 1 and 5).
 *
 * For query head h in KV group g: local groups see tokens [0, sinks) and
 * [n_ctx - window, n_ctx) (a union); retrieval and routed groups see
 * sel_idx[b,g,0:sel_count[b,g]].  out[b,h,:] = sum_j pi_j v_j with
 * pi = softmax(q[b,h] . k_j / sqrt(d)) over that set, accumulated in fp32.
 * The GQA heads of a group share every gathered key/value row.  Reads q,
 * k_cache, v_cache, sel_idx, sel_count; writes out.  Needs a workspace.
 */
int32_t sparse_attn_decode(const sa_params* params, const sa_buffers* bufs,
                           void* workspace, size_t* workspace_bytes,
                           void* hip_stream);

/*
 * sparse_attn_prefill_chunked - pyramid-selection prefill forward
 * (Lighthouse summary, 2C).  For every block of q_block level-0 queries,
 * each query i attends to the block's selected entries (rows of k_cache /
 * v_cache for level 0, of pyr_k / pyr_v above) plus the block's own level-0
 * keys up to and including i, with scale 1/sqrt(d); the fp32 result is
 * written to out row i.  Requires n_q_heads == n_kv_heads, dtype bf16,
 * head_dim 128, q_block 128, block_top_k <= 8192 and n_ctx < 2^23
 * (SA_ERR_UNSUPPORTED otherwise).  blk_idx holds flat ids as
 * SA_SEL_PYRAMID_TOPK writes them; an id outside [0, n_ctx + coarse entries)
 * is never dereferenced: level-0 row 0 is read in its place, so its
 * contribution is unspecified.  Needs a workspace.
 */
int32_t sparse_attn_prefill_chunked(const sa_params* params, const sa_buffers* bufs,
                                    void* workspace, size_t* workspace_bytes,
                                    void* hip_stream);

/* Human-readable name of a status code (static string). */
const char* sparse_attn_status_string(int32_t status);

/* SPARSE_ATTN_VERSION of the built library. */
int32_t sparse_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
