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
 *    the library never allocates or frees memory and keeps no pointer after a
 *    call returns.  Its only global state is the device address of the
 *    static scratch array of sparse_attn_decode_noalloc, looked up once per
 *    device.  Calls on different streams with disjoint output and workspace
 *    buffers may run concurrently, with one exception: two top-p / top-k
 *    selections (SA_SEL_TOPP, SA_SEL_TOPK, SA_SEL_TOPK_BY_SCORE) must not
 *    overlap on one device.  Each keeps the workgroups of a row waiting for
 *    one another and is sized to be resident on its own; two at once can
 *    hold every slot with half-resident rows, and their bounded waits then
 *    end in a reported failure (sel_count -1), not a hang.
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

#define SPARSE_ATTN_VERSION 6

/* Size of the static device scratch array behind sparse_attn_decode_noalloc
 * (one per GPU the library runs on, held until the process ends). */
#define SPARSE_ATTN_NOALLOC_SCRATCH_BYTES (8u << 20)

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
  SA_SEL_PYRAMID_TOPK = 3,  /* per query block: joint top-K over levels       */
  SA_SEL_ROUTE2_PREFILL = 4,/* routed groups, prefill: per query block (chunk) */
  SA_SEL_TOPK_BY_SCORE = 5  /* retrieval groups: top_k, listed by index score   */
} sa_select_mode;

/* OR'ed into SA_SEL_TOPP, SA_SEL_TOPK or SA_SEL_TOPK_BY_SCORE: the decode
 * step's index append is fused into the selection.  Before ranking, the call
 * projects the query heads of every selecting row into q_idx and token
 * n_ctx - 1 into k_idx, with the same bits as sparse_attn_index_build(
 * SA_IDX_LOWRANK, n_ctx - 1, n_ctx) (which then need not be called).  Reads
 * q_pre, k_pre, proj_q and proj_k as well; bf16 caches only
 * (SA_ERR_UNSUPPORTED otherwise); q_pre, k_pre, proj_q, proj_k and q_idx
 * 16-byte aligned.  With any other mode it gives SA_ERR_INVALID_ARG. */
#define SA_SEL_APPEND 0x100

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
  int32_t per_head_sets;/* 0: one set per KV group, shared by its G query heads;
                         * 1: one set per query head (see below)               */
  float s2o_tau;        /* decode: > 0 turns on the monotone-gain early stop of
                         * retrieval groups (see sparse_attn_decode); 0: off   */
} sa_params;

/*
 * Per-query-head sets (per_head_sets = 1; the "Full Attention Strikes Back"
 * summary speaks of per-head sparse attention, read here as every query head
 * selecting for itself).  SA_SEL_TOPP / SA_SEL_TOPK and SA_SEL_ROUTE2 then
 * treat each query head as a group of one: a retrieval head ranks tokens with
 * its own q_idx row, a routed head routes with its own query, against the
 * index keys or summaries of its KV group h / G.  sel_idx is [B,Hq,n_cap] and
 * sel_count [B,Hq], and sparse_attn_decode reads them per query head.  With
 * bf16 caches, n_ctx < 2^24 and no early stop, the decode still gathers
 * each row once per KV group: it merges the group's heads' lists into one
 * (ascending, each position tagged with the heads that chose it) in its
 * workspace and masks every head to its own set; otherwise each head is
 * decoded alone.  Labels must still be equal inside a GQA group, and
 * n_q_heads <= 64.  The index build is the same in both modes.
 */

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
                        /* ([B,Hq,n_cap] with per_head_sets)                   */
  int32_t* sel_count;   /* [B,Hkv] number of valid entries in sel_idx ([B,Hq]) */
  int32_t* blk_idx;     /* [B,H,ceil(N/q_block),K] flat entry ids per block    */
  int32_t* blk_count;   /* [B,H,ceil(N/q_block)]                               */
  float* out;           /* [B,Hq,d] decode | [B,H,N,d] prefill, fp32           */
  /* pyramid prefill training pass (sparse_attn_prefill_backward)              */
  const float* grad_out; /* [B,H,N,d] fp32   gradient of the loss w.r.t. out    */
  float* lse;           /* [B,H,N] fp32      per query: log sum_j exp(q.k_j/sqrt d) */
  float* grad_q;        /* [B,H,N,d] fp32    gradient w.r.t. level-0 Q           */
  float* grad_k;        /* [B,H,N,d] fp32    gradient w.r.t. level-0 K           */
  float* grad_v;        /* [B,H,N,d] fp32    gradient w.r.t. level-0 V           */
  /* coarse-query outputs of the pyramid prefill (sparse_attn_prefill_coarse)   */
  float* out_pyr;       /* [B,H,Nc,d] fp32   one row per coarse entry, as pyr_q  */
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
 * SA_SEL_TOPK_BY_SCORE ("S2O" summary, Methodology 1-2: candidates visited in
 *   descending estimated importance): the SA_SEL_TOPK set, written to sel_idx
 *   in (logit desc, position asc) order instead of ascending - the visit
 *   order of the early-stop decode.  Needs top_k <= 8192
 *   (SA_ERR_UNSUPPORTED).
 * SA_SEL_ROUTE2_PREFILL (HGA summary, Core mechanism items 1-2, routing
 *   while prefilling): for each routed group and every query block of
 *   chunk = 128 queries (block beta holds positions 128 beta .. t, t its last
 *   position), qbar = mean of the block's post-RoPE query rows q[b,h,i] over
 *   the group's heads; the block then routes as SA_SEL_ROUTE2 does at
 *   position t (kappa = beta), and its list - sink chunks, local chunks and
 *   routed groups, all before the block - is written ascending to
 *   blk_idx[b,g,beta,:] with its length in blk_count[b,g,beta];
 *   sparse_attn_prefill_chunked with levels = 1 then adds each query's own
 *   causal part of the block.  q is [B,Hq,n_ctx,d]; blk_idx is
 *   [B,Hkv,ceil(n_ctx/128),block_top_k].  Needs chunk == 128 and
 *   per_head_sets == 0 (SA_ERR_UNSUPPORTED) and block_top_k >= (sink_chunks +
 *   local_chunks) * chunk + top_chunks * top_groups * group (SA_ERR_CAPACITY).
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
 * The GQA heads of a group share every gathered key/value row.  With
 * per_head_sets, head h sees sel_idx[b,h,0:sel_count[b,h]] (local heads as
 * above) over the rows of KV group h / G.
 * With s2o_tau > 0 ("S2O" summary, Methodology 2-3: monotone-gain early
 * stop), retrieval groups instead read sel_idx as candidates in visit order
 * (SA_SEL_TOPK_BY_SCORE; at most 8192 are read): each head attends first
 * over the local rule's tokens (sinks + window), then over the candidates
 * outside them in blocks of 64 in list order, and after each block stops
 * when the block's attention mass falls below s2o_tau times the mass
 * attended before it (that block is kept).  Needs dtype bf16 and sinks +
 * window >= 1.  Reads q,
 * k_cache, v_cache, sel_idx, sel_count; writes out.  A selecting group whose
 * sel_count is negative (a selection that reported failure) gets NaN in
 * every output of its query heads (with per_head_sets: a head whose count
 * is negative gets NaN in its own outputs).  Needs a workspace; no part of it has to
 * start at zero.
 */
int32_t sparse_attn_decode(const sa_params* params, const sa_buffers* bufs,
                           void* workspace, size_t* workspace_bytes,
                           void* hip_stream);

/*
 * sparse_attn_decode_noalloc - sparse_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, validation, kernels and
 * results as sparse_attn_decode, without the workspace arguments: the
 * workspace is carved from a static device array of
 * SPARSE_ATTN_NOALLOC_SCRATCH_BYTES on the current device (the stream must
 * belong to it).  The call allocates nothing; the first call on a device
 * looks up that device's copy of the array.  Returns SA_ERR_WORKSPACE when
 * the workspace sparse_attn_decode would need is larger than the array, and
 * SA_ERR_HIP when the array's address cannot be obtained.  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other host threads) race and give undefined results.  The array
 * keeps the last call's contents; nothing in it needs to start at zero.
 */
int32_t sparse_attn_decode_noalloc(const sa_params* params, const sa_buffers* bufs,
                                   void* hip_stream);

/*
 * sparse_attn_prefill_chunked - pyramid-selection prefill forward
 * (Lighthouse summary, 2C).  For every block of q_block level-0 queries,
 * each query i attends to the block's selected entries (rows of k_cache /
 * v_cache for level 0, of pyr_k / pyr_v above) plus the block's own level-0
 * keys up to and including i, with scale 1/sqrt(d); the fp32 result is
 * written to out row i.  With levels = 1 the heads may be grouped (GQA):
 * blk_idx / blk_count then belong to the KV heads ([B,Hkv,...]) and the G
 * query heads of a group share its lists and rows (the layout
 * SA_SEL_ROUTE2_PREFILL writes); otherwise n_q_heads == n_kv_heads.
 * Requires dtype bf16,
 * head_dim 128, q_block 128, block_top_k <= 8192 and n_ctx < 2^23
 * (SA_ERR_UNSUPPORTED otherwise).  blk_idx holds flat ids as
 * SA_SEL_PYRAMID_TOPK writes them; an id outside [0, n_ctx + coarse entries)
 * is never dereferenced: level-0 row 0 is read in its place, so its
 * contribution is unspecified.  When lse is not NULL it also receives, per
 * query, the natural log of the softmax denominator sum_j exp(q.k_j /
 * sqrt(d)) (what sparse_attn_prefill_backward reads).  Needs a workspace.
 */
int32_t sparse_attn_prefill_chunked(const sa_params* params, const sa_buffers* bufs,
                                    void* workspace, size_t* workspace_bytes,
                                    void* hip_stream);

/*
 * sparse_attn_prefill_coarse - the coarse queries of the pyramid-selection
 * prefill (Lighthouse summary, 2A: Q, K and V are aggregated symmetrically;
 * 2C: the gathered entries attend as one subsequence and each output is
 * scattered back to where its entry came from).  For every block of q_block
 * level-0 positions and every level l = 1 .. levels-1, each coarse query
 * entry j of level l whose span lies in the block (rows of pyr_q) attends to
 * the block's selected entries (as in sparse_attn_prefill_chunked) plus the
 * block's own level-l entries up to and including j (rows of pyr_k / pyr_v),
 * with scale 1/sqrt(d); the fp32 result goes to row j of level l in out_pyr
 * (the pyr_q layout).  Level-0 outputs are sparse_attn_prefill_chunked's;
 * how a model combines the levels is left to the caller.  Reads pyr_q,
 * pyr_k, pyr_v, k_cache, v_cache, blk_idx, blk_count; writes out_pyr.  Same
 * requirements as sparse_attn_prefill_chunked, with n_q_heads == n_kv_heads;
 * levels = 1 has no coarse queries and returns SA_OK with nothing written.
 * No workspace; no backward (sparse_attn_prefill_backward covers the level-0
 * outputs only).
 */
int32_t sparse_attn_prefill_coarse(const sa_params* params, const sa_buffers* bufs,
                                   void* hip_stream);

/*
 * sparse_attn_prefill_backward - gradients of the pyramid-selection prefill
 * (Lighthouse summary, 2B-2C: the selection is discrete and receives no
 * gradient; gradients pass through the gather, the attention and the scatter
 * back; 2A: a level-l entry is the mean of the p^l level-0 rows it covers).
 *
 * For a loss L with dL/d(out) = grad_out, writes dL/dQ, dL/dK and dL/dV of the
 * level-0 Q, K and V of sparse_attn_prefill_chunked, its selection (blk_idx,
 * blk_count) held fixed: per block, with P the softmax weights and a = q.k /
 * sqrt(d), dV_j += P_ij dO_i, dA_ij = P_ij (dO_i.v_j - dO_i.o_i), dQ_i = sum_j
 * dA_ij k_j / sqrt(d), dK_j += dA_ij q_i / sqrt(d); the gradient of a coarse
 * entry at level l goes to each level-0 row it covers divided by p^l (the
 * stored rounding of a level counts as the identity).  Only level-0 queries
 * attend, so the coarse Q levels get no gradient.
 *
 * Reads q, k_cache, v_cache, pyr_k, pyr_v (levels > 1), blk_idx, blk_count,
 * out and lse as sparse_attn_prefill_chunked wrote them (pass lse to the
 * forward call), and grad_out; writes grad_q, grad_k, grad_v.  Same
 * requirements as the forward plus n_q_heads == n_kv_heads
 * (SA_ERR_UNSUPPORTED).  The lists may come in any order, but they must have
 * the shape the pyramid selection gives them: distinct visible ids, each
 * entry chosen from the first block that sees it through a last block and by
 * none after.  A head whose lists break this (or hold a negative count or an
 * id outside the pyramid) gets NaN in every gradient row.  Deterministic:
 * every sum is taken in a fixed order.  Needs a workspace of about
 * B * H * (N + ceil(N/128) * block_top_k) * d * 8 bytes (per-block partial
 * gradients of the chosen entries, reduced per entry in block order); no
 * part of it has to start at zero.
 */
int32_t sparse_attn_prefill_backward(const sa_params* params, const sa_buffers* bufs,
                                     void* workspace, size_t* workspace_bytes,
                                     void* hip_stream);

/*
 * sparse_attn_prefill_heads - head-split prefill forward ("Full Attention
 * Strikes Back" summary, Methodology item 1 and Results: local heads window
 * their prefill, retrieval heads keep the whole cache; AoH summary,
 * Methodology item 4).  Every query position i = 0 .. n_ctx - 1 of query head
 * h attends, with scale 1/sqrt(d), over the keys of KV group h / G that its
 * label allows: a local head sees positions [0, sinks) and [i - window + 1,
 * i] (a union, clipped to [0, i]) - what a decode query would see with a
 * cache of i + 1 keys; a retrieval or routed head sees [0, i] (dense causal).
 * q is [B,Hq,n_ctx,d] (post-RoPE), k_cache / v_cache [B,Hkv,n_cap,d] with
 * keys 0 .. n_ctx - 1 filled, out [B,Hq,n_ctx,d] fp32.  Requires dtype bf16,
 * head_dim 128, n_q_heads <= 128 and n_ctx < 2^23 (SA_ERR_UNSUPPORTED
 * otherwise); sinks >= 0, window >= 0 and sinks + window >= 1 when some head
 * is local.  No workspace; q_block and the selection fields are not used.
 */
int32_t sparse_attn_prefill_heads(const sa_params* params, const sa_buffers* bufs,
                                  void* hip_stream);

/*
 * Tiered K/V store of the routed decode (HGA summary, Memory architecture:
 * the whole K/V history in host RAM - cold -, a bounded LRU cache of
 * recently routed blocks in device memory - warm -, the summaries and the
 * always-visible windows in device memory - hot; Core mechanism item 4: the
 * routed groups' token-level K/V rows are brought from host RAM).
 *
 * The device tier of each (sequence, KV group) holds dev_rows = hot_rows +
 * warm_slots * group rows of K (and of V), hot_rows = (sink_chunks +
 * local_chunks + 1) * chunk: rows [0, sink_chunks * chunk) are the sink
 * positions themselves, the next (local_chunks + 1) * chunk rows a ring of
 * the last chunks (position p at row sink_chunks * chunk + p mod that ring),
 * and warm slot s the rows of one routing group.  The caller keeps the cold
 * store (every cached token) and the hot rows up to date; the library keeps
 * the warm slots.
 */
typedef struct sa_tier {
  const void* cold_k;    /* pinned host memory [B,Hkv,n_cap,d]: every cached token's K */
  const void* cold_v;    /* (allocated with hipHostMalloc, e.g. torch pin_memory)      */
  void* dev_k;           /* device [B,Hkv,dev_rows,d]                                  */
  void* dev_v;
  int32_t warm_slots;    /* slots per (b, KV group); >= top_chunks * top_groups, <= 4096 */
  int32_t step;          /* this call's stamp: larger than every earlier call's        */
  int32_t* slot_group;   /* device [B,Hkv,warm_slots] group held, -1 empty (start: -1) */
  int32_t* slot_stamp;   /* device [B,Hkv,warm_slots] step of last use (start: 0)      */
  int32_t* stats;        /* device [B,Hkv,2] or NULL: this call's hits and misses      */
  int32_t* rows;         /* device [B,Hkv,dev_rows]: the lists as rows of the device tier */
} sa_tier;

/*
 * sparse_attn_tier_fetch - serve the routed lists of one decode step from
 * the tiers.  For every routed KV group, after SA_SEL_ROUTE2 wrote its list
 * (ascending positions) to sel_idx / sel_count: the distinct routing groups
 * of the list's routed part (positions in [sink_chunks * chunk, (kappa -
 * local_chunks) * chunk), kappa = (n_ctx - 1) / chunk) that no warm slot
 * holds are copied from the cold store into slots - empty slots first, then
 * the least recently used slot the step does not need (ties: lower slot),
 * missing groups in ascending order - and every slot the step uses takes
 * the stamp `step`; then the list is written to `rows` (same counts) as rows
 * of the device tier.  sparse_attn_decode with k_cache / v_cache = dev_k /
 * dev_v, sel_idx = rows and n_ctx = n_cap = dev_rows then computes the same
 * outputs as over the whole cache.  Needs
 * every head routed, per_head_sets == 0, chunk a multiple of group, and
 * lists of at most 8192 entries (SA_ERR_UNSUPPORTED otherwise); cold
 * pointers the device cannot reach give SA_ERR_INVALID_ARG.  Calls that
 * share tables must not overlap.  No workspace.
 */
int32_t sparse_attn_tier_fetch(const sa_params* params, const sa_buffers* bufs,
                               const sa_tier* tier, void* hip_stream);

/* Human-readable name of a status code (static string). */
const char* sparse_attn_status_string(int32_t status);

/* SPARSE_ATTN_VERSION of the built library. */
int32_t sparse_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
