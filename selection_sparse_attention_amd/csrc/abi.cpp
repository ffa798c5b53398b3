// C ABI of the sparse attention library: argument validation, workspace
// sizing and carving, and kernel launch on the caller's stream.  Nothing here
// allocates, frees, copies to the host or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "../../include/sparse_attn.h"
#include "abi_internal.hpp"
#include "args.hpp"

namespace {

using sa::GroupList;

constexpr size_t kAlign = 256;
constexpr size_t kMinWorkspace = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Carves consecutive, 256-byte aligned pieces out of a workspace (or, with a
// null base, only measures them).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + count * sizeof(T));
    return p;
  }
  size_t size() const { return off < kMinWorkspace ? kMinWorkspace : off; }
};

// Labels of the KV groups; SA_OK when every group's heads agree.
int32_t group_kinds(const sa_params* p, int8_t* kind_of_group) {
  if (!p->head_kind) return SA_ERR_INVALID_ARG;
  const int G = p->n_q_heads / p->n_kv_heads;
  for (int g = 0; g < p->n_kv_heads; ++g) {
    const int8_t k0 = p->head_kind[g * G];
    if (k0 < SA_HEAD_LOCAL || k0 > SA_HEAD_ROUTED) return SA_ERR_INVALID_ARG;
    for (int h = 1; h < G; ++h)
      if (p->head_kind[g * G + h] != k0) return SA_ERR_INVALID_ARG;
    kind_of_group[g] = k0;
  }
  return SA_OK;
}

GroupList groups_of_kind(const sa_params* p, const int8_t* kinds, int kind) {
  GroupList gl{};
  gl.n = 0;
  for (int g = 0; g < p->n_kv_heads; ++g)
    if (kinds[g] == kind) gl.ids[gl.n++] = g;
  return gl;
}

// The units that select and attend together: the KV groups (their G query
// heads share one set), or, with per-head sets, every query head alone (a
// group of one head; kv_div of them per KV group).
struct SelGroups {
  int n;                        // units per sequence
  int G;                        // query heads per unit
  int kv_div;                   // units per KV group
  int8_t kind[sa::kMaxGroups];  // label of each unit
};

int32_t sel_groups(const sa_params* p, SelGroups* u) {
  int8_t kinds[sa::kMaxGroups];
  int32_t st = group_kinds(p, kinds);
  if (st) return st;
  const int G = p->n_q_heads / p->n_kv_heads;
  if (p->per_head_sets != 0 && p->per_head_sets != 1) return SA_ERR_INVALID_ARG;
  if (!p->per_head_sets) {
    u->n = p->n_kv_heads; u->G = G; u->kv_div = 1;
    for (int g = 0; g < p->n_kv_heads; ++g) u->kind[g] = kinds[g];
    return SA_OK;
  }
  if (p->n_q_heads > sa::kMaxGroups) return SA_ERR_UNSUPPORTED;
  u->n = p->n_q_heads; u->G = 1; u->kv_div = G;
  for (int h = 0; h < p->n_q_heads; ++h) u->kind[h] = kinds[h / G];
  return SA_OK;
}

GroupList units_of_kind(const SelGroups& u, int kind) {
  GroupList gl{};
  gl.n = 0;
  for (int g = 0; g < u.n; ++g)
    if (u.kind[g] == kind) gl.ids[gl.n++] = g;
  return gl;
}

// Checks shared by every entry point.
int32_t check_common(const sa_params* p, const sa_buffers* b) {
  if (!p || !b) return SA_ERR_INVALID_ARG;
  if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1) return SA_ERR_INVALID_ARG;
  if (p->n_q_heads % p->n_kv_heads != 0) return SA_ERR_INVALID_ARG;
  if (p->n_ctx < 1 || p->n_cap < p->n_ctx) return SA_ERR_INVALID_ARG;
  if (p->dtype != SA_BF16 && p->dtype != SA_FP32) return SA_ERR_INVALID_ARG;
  if (p->head_dim != 64 && p->head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (p->n_kv_heads > sa::kMaxGroups) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

int32_t workspace_gate(void* ws, size_t* ws_bytes, size_t need) {
  if (!ws_bytes) return SA_ERR_INVALID_ARG;
  if (!ws) { *ws_bytes = need; return 1; }          // size query
  if (*ws_bytes < need) return SA_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return SA_ERR_INVALID_ARG;
  return SA_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? SA_OK : SA_ERR_HIP; }

int pow_int(int b, int e) {
  int r = 1;
  for (int i = 0; i < e; ++i) r *= b;
  return r;
}

// ---------------------------------------------------------------- pyramid
struct PyrGeom {
  int N, L, p, top_span, Nc, Nt, nblk;
  int off[16];   // flat offsets of each level
};

// allow_gqa: one level (no pyramid), the lists belonging to the KV heads
int32_t pyramid_geom(const sa_params* p, PyrGeom* g, bool allow_gqa = false) {
  if (p->levels < 1 || p->levels > 8 || p->factor < 2) return SA_ERR_INVALID_ARG;
  if (p->n_q_heads != p->n_kv_heads && !(allow_gqa && p->levels == 1)) return SA_ERR_INVALID_ARG;
  const int64_t span = [&] { int64_t s = 1; for (int i = 1; i < p->levels; ++i) s *= p->factor; return s; }();
  if (span > 256) return SA_ERR_UNSUPPORTED;
  if (p->n_ctx % span) return SA_ERR_INVALID_ARG;
  g->N = p->n_ctx; g->L = p->levels; g->p = p->factor; g->top_span = (int)span;
  int o = 0, m = p->n_ctx;
  g->Nc = 0;
  for (int l = 0; l < p->levels; ++l) {
    g->off[l] = o;
    o += m;
    if (l > 0) g->Nc += m;
    m /= p->factor;
  }
  g->Nt = o;
  g->nblk = p->q_block > 0 ? (p->n_ctx + p->q_block - 1) / p->q_block : 0;
  return SA_OK;
}

// ---------------------------------------------------------------- select ws
struct SelectWs {
  uint32_t* hist_c; double* hist_m; uint32_t* ctl; uint32_t* slot_a; uint64_t* slot_b;
  uint32_t* cand; size_t bytes;
};

// The regions that must be zero when a call starts (histograms, control
// words, flags; returned to zero by every call) come first, and their sizes
// depend on the number of rows only; the candidate regions (a tile of keys
// per workgroup, written before they are read) come last.
SelectWs carve_select(void* ws, int rows, int64_t cand_stride) {
  SelectWs s{};
  Carver c(ws);
  s.hist_c = c.take<uint32_t>((size_t)rows * 3 * 4096);
  s.hist_m = c.take<double>((size_t)rows * 3 * 4096);
  s.ctl = c.take<uint32_t>((size_t)rows * sa::kCtlWords);
  s.slot_a = c.take<uint32_t>((size_t)rows * sa::kMaxSelW);
  s.slot_b = c.take<uint64_t>((size_t)rows * sa::kMaxSelW);
  s.cand = c.take<uint32_t>((size_t)rows * cand_stride);
  s.bytes = c.size();
  return s;
}

// Polls per cross-workgroup wait of the selector: about a second at the
// default.  SPARSE_ATTN_SPIN_LIMIT overrides it (a negative value fails every
// wait at once: a diagnostic for the failure path).
int select_spin_limit() {
  const char* e = std::getenv("SPARSE_ATTN_SPIN_LIMIT");
  if (e && *e) return std::atoi(e);
  return 1 << 20;
}

// ---------------------------------------------------------------- decode ws
constexpr int kDecodeTps = 256;           // fp32 caches: list entries per split
constexpr int kDecodeMinChunk = 64;       // bf16 caches: smallest work item (list entries)
constexpr int kMaxDecodeItems = 8192;     // bf16 caches: work items one launch may hold
constexpr int kMaxDecodeSplits = 8192;     // contexts up to 2M tokens

// Compute units of the current device (a runtime query on every call: the
// library keeps no state between calls).
int compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  return n;
}

int decode_max_count(const sa_params* p, const SelGroups& u) {
  const int8_t* kinds = u.kind;
  int mc = 0;
  for (int g = 0; g < u.n; ++g) {
    int c;
    if (kinds[g] == SA_HEAD_LOCAL) {
      const int64_t sw = (int64_t)p->sinks + p->window;
      c = (int)(sw < p->n_ctx ? sw : p->n_ctx);
    } else {
      c = p->n_ctx;
    }
    mc = c > mc ? c : mc;
  }
  return mc;
}

}  // namespace

namespace sa {

// The decode entry point's work, shared with the entry point that takes its
// workspace from the library's static scratch array.
int32_t decode_entry(const sa_params* p, const sa_buffers* b, void* ws, size_t* ws_bytes,
                     void* stream) {
  int32_t st = check_common(p, b);
  if (st) return st;
  SelGroups u;
  if ((st = sel_groups(p, &u))) return st;
  const int G = u.G;
  if (G != 1 && G != 2 && G != 4 && G != 8) return SA_ERR_UNSUPPORTED;
  bool any_local = false, any_list = false;
  uint64_t local_mask = 0, s2o_mask = 0;
  const bool s2o = p->s2o_tau > 0.f;
  if (std::isnan(p->s2o_tau) || p->s2o_tau < 0.f) return SA_ERR_INVALID_ARG;
  GroupList s2o_units{};
  for (int g = 0; g < u.n; ++g) {
    if (u.kind[g] == SA_HEAD_LOCAL) { any_local = true; local_mask |= 1ull << g; }
    else any_list = true;
    if (s2o && u.kind[g] == SA_HEAD_RETRIEVAL) { s2o_mask |= 1ull << g; s2o_units.ids[s2o_units.n++] = g; }
  }
  // an early-stop group's first pass is the local rule, run by the split kernels
  local_mask |= s2o_mask;
  if ((any_local || s2o_mask) && (p->sinks < 0 || p->window < 0 || (int64_t)p->sinks + p->window < 1))
    return SA_ERR_INVALID_ARG;
  if (s2o_mask && p->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  int tps = kDecodeTps, max_splits, target_items = 0;
  size_t n_partial;
  if (p->dtype == SA_BF16) {
    // work items: the step's visible tokens spread over one item per
    // workgroup slot (two per compute unit, one for 8-head groups, whose
    // workgroups use a whole unit's registers); the plan itself is made on
    // the device
    const int groups = p->batch * u.n;
    target_items = (G > 4 ? 1 : 2) * compute_units();
    max_splits = target_items + groups;        // bound on the item count
    if (max_splits > kMaxDecodeItems) return SA_ERR_UNSUPPORTED;
    n_partial = (size_t)max_splits * G * (p->head_dim + 2);
  } else {
    const int max_count = decode_max_count(p, u);
    max_splits = (max_count + tps - 1) / tps;
    if (max_splits > kMaxDecodeSplits) return SA_ERR_UNSUPPORTED;
    n_partial = (size_t)p->batch * p->n_q_heads * max_splits * (p->head_dim + 2);
  }
  // per-head sets on the matrix-core path: each KV group's heads share one
  // union list with head bits, so every row is gathered once for the group
  // (decoded as KV groups of G heads with per-head masks)
  const int Gkv = p->n_q_heads / p->n_kv_heads;
  const bool head_union = p->per_head_sets && p->dtype == SA_BF16 && !s2o_mask && Gkv > 1 &&
                          any_list && p->n_ctx <= sa::kUnionMaxN;
  SelGroups ug = u;
  if (head_union) {
    ug.n = p->n_kv_heads; ug.G = Gkv; ug.kv_div = 1;
    for (int g = 0; g < p->n_kv_heads; ++g) ug.kind[g] = u.kind[g * Gkv];
    local_mask = 0;
    for (int g = 0; g < ug.n; ++g)
      if (ug.kind[g] == SA_HEAD_LOCAL) local_mask |= 1ull << g;
    const int groups = p->batch * ug.n;
    target_items = (Gkv > 4 ? 1 : 2) * compute_units();
    max_splits = target_items + groups;
    if (max_splits > kMaxDecodeItems) return SA_ERR_UNSUPPORTED;
    n_partial = (size_t)max_splits * Gkv * (p->head_dim + 2);
  }
  Carver c(ws);
  float* partial = c.take<float>(n_partial);
  int2* plan = (p->dtype == SA_BF16) ? c.take<int2>((size_t)p->batch * ug.n) : nullptr;
  float* s2o_state = s2o_mask ? c.take<float>((size_t)p->batch * u.n * G * (p->head_dim + 2)) : nullptr;
  int32_t* union_idx = head_union ? c.take<int32_t>((size_t)p->batch * p->n_kv_heads * p->n_cap) : nullptr;
  int32_t* union_count = head_union ? c.take<int32_t>((size_t)p->batch * p->n_kv_heads) : nullptr;
  const int mask_words = (p->n_ctx + 3) / 4;
  const int n_slices = (p->n_ctx + sa::kUnionSlice - 1) / sa::kUnionSlice;
  uint32_t* union_masks = head_union ? c.take<uint32_t>((size_t)p->batch * p->n_kv_heads * mask_words) : nullptr;
  int32_t* slice_count = head_union ? c.take<int32_t>((size_t)p->batch * p->n_kv_heads * n_slices) : nullptr;

  if ((st = workspace_gate(ws, ws_bytes, c.size()))) return st < 0 ? st : SA_OK;
  if (!b->q || !b->k_cache || !b->v_cache || !b->out) return SA_ERR_INVALID_ARG;
  if (any_list && (!b->sel_idx || !b->sel_count)) return SA_ERR_INVALID_ARG;
  if (!aligned16(b->q) || !aligned16(b->k_cache) || !aligned16(b->v_cache)) return SA_ERR_INVALID_ARG;
  sa::DecodeArgs a{};
  a.q = b->q; a.k = b->k_cache; a.v = b->v_cache; a.sel_idx = b->sel_idx; a.sel_count = b->sel_count;
  a.out = b->out; a.partial = partial;
  a.B = p->batch; a.Hq = p->n_q_heads; a.Hkv = u.n; a.n = p->n_ctx; a.n_cap = p->n_cap;
  a.G = G; a.kv_div = u.kv_div;
  a.sinks = p->sinks; a.window = p->window; a.tps = tps; a.max_splits = max_splits;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  a.local_mask = local_mask;
  a.target_items = target_items;
  a.min_chunk = kDecodeMinChunk;
  a.plan = plan;
  a.s2o_mask = s2o_mask;
  a.s2o_state = s2o_state;
  a.s2o_tau = p->s2o_tau;
  a.s2o = s2o_units;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (head_union) {
    sa::HeadUnionArgs ua{};
    ua.sel_idx = b->sel_idx; ua.sel_count = b->sel_count;
    ua.union_idx = union_idx; ua.union_count = union_count;
    ua.B = p->batch; ua.Hq = p->n_q_heads; ua.Hkv = p->n_kv_heads; ua.G = Gkv;
    ua.n = p->n_ctx; ua.n_cap = p->n_cap;
    ua.masks = union_masks; ua.slice_count = slice_count;
    ua.mask_words = mask_words; ua.n_slices = n_slices;
    ua.groups.n = 0;
    for (int g = 0; g < ug.n; ++g)
      if (ug.kind[g] != SA_HEAD_LOCAL) ua.groups.ids[ua.groups.n++] = g;
    if ((st = hip_status(sa::launch_head_union(ua, hs)))) return st;
    a.sel_idx = union_idx; a.sel_count = union_count;
    a.Hkv = ug.n; a.G = Gkv; a.kv_div = 1;
    a.head_masks = 1; a.head_count = b->sel_count;
  }
  if ((st = hip_status(sa::launch_decode(a, p->dtype, p->head_dim, hs)))) return st;
  if (!s2o_mask) return SA_OK;
  return hip_status(sa::launch_decode_s2o(a, p->head_dim, hs));
}

}  // namespace sa

extern "C" {

const char* sparse_attn_status_string(int32_t s) {
  switch (s) {
    case SA_OK: return "SA_OK";
    case SA_ERR_INVALID_ARG: return "SA_ERR_INVALID_ARG";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED";
    case SA_ERR_WORKSPACE: return "SA_ERR_WORKSPACE";
    case SA_ERR_CAPACITY: return "SA_ERR_CAPACITY";
    case SA_ERR_HIP: return "SA_ERR_HIP";
    default: return "SA_ERR_UNKNOWN";
  }
}

int32_t sparse_attn_version(void) { return SPARSE_ATTN_VERSION; }

int32_t sparse_attn_index_build(const sa_params* p, const sa_buffers* b, int32_t mode,
                                int32_t t_begin, int32_t t_end, void* stream) {
  int32_t st = check_common(p, b);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == SA_IDX_PYRAMID) {
    PyrGeom pg;
    if ((st = pyramid_geom(p, &pg))) return st;
    if (t_begin != 0 || t_end != p->n_ctx) return SA_ERR_INVALID_ARG;
    if (!b->q || !b->k_cache || !b->v_cache || !b->pyr_scores) return SA_ERR_INVALID_ARG;
    if (p->levels > 1 && (!b->pyr_q || !b->pyr_k || !b->pyr_v)) return SA_ERR_INVALID_ARG;
    sa::PyramidArgs a{};
    a.q = b->q; a.k = b->k_cache; a.v = b->v_cache;
    a.pq = b->pyr_q; a.pk = b->pyr_k; a.pv = b->pyr_v; a.scores = b->pyr_scores;
    a.B = p->batch; a.H = p->n_q_heads; a.N = p->n_ctx; a.levels = p->levels; a.factor = p->factor;
    a.Nc = pg.Nc; a.Nt = pg.Nt; a.top_span = pg.top_span;
    for (int l = 0; l < 8; ++l) {
      a.soff[l] = l < p->levels ? pg.off[l] : 0;
      a.coff[l] = l < p->levels && l > 0 ? pg.off[l] - p->n_ctx : 0;
    }
    return hip_status(sa::launch_pyramid(a, p->dtype, p->head_dim, s));
  }
  int8_t kinds[sa::kMaxGroups];
  if ((st = group_kinds(p, kinds))) return st;
  if (t_begin < 0 || t_end <= t_begin || t_end > p->n_cap) return SA_ERR_INVALID_ARG;
  const int G = p->n_q_heads / p->n_kv_heads;
  if (mode == SA_IDX_LOWRANK) {
    if (p->r != 16) return SA_ERR_UNSUPPORTED;
    GroupList gl = groups_of_kind(p, kinds, SA_HEAD_RETRIEVAL);
    if (gl.n == 0) return SA_OK;
    if (!b->k_pre || !b->proj_k || !b->k_idx) return SA_ERR_INVALID_ARG;
    if (b->q_pre && (!b->proj_q || !b->q_idx)) return SA_ERR_INVALID_ARG;
    if (!aligned16(b->k_pre) || !aligned16(b->k_idx)) return SA_ERR_INVALID_ARG;
    sa::IndexLowrankArgs a{};
    a.k_pre = b->k_pre; a.q_pre = b->q_pre; a.proj_q = b->proj_q; a.proj_k = b->proj_k;
    a.k_idx = b->k_idx; a.q_idx = b->q_idx;
    a.B = p->batch; a.Hq = p->n_q_heads; a.Hkv = p->n_kv_heads; a.n_cap = p->n_cap; a.G = G;
    a.t0 = t_begin; a.t1 = t_end; a.groups = gl;
    a.tokens_per_wg = 2048;      // a whole number of the kernel's steps for every shape
    return hip_status(sa::launch_index_lowrank(a, p->dtype, p->head_dim, s));
  }
  if (mode == SA_IDX_CHUNK_SUMMARY) {
    if (p->chunk < 1 || p->group < 1 || p->chunk % p->group) return SA_ERR_INVALID_ARG;
    if (!(p->rope_base > 0.f)) return SA_ERR_INVALID_ARG;
    GroupList gl = groups_of_kind(p, kinds, SA_HEAD_ROUTED);
    if (gl.n == 0) return SA_OK;
    if (!b->k_pre || !b->chunk_sum || !b->group_sum) return SA_ERR_INVALID_ARG;
    sa::SummaryArgs a{};
    a.k_pre = b->k_pre; a.chunk_sum = b->chunk_sum; a.group_sum = b->group_sum;
    a.B = p->batch; a.Hkv = p->n_kv_heads; a.n_cap = p->n_cap; a.chunk = p->chunk; a.group = p->group;
    // spans whose last token lies in [t_begin, t_end): span c ends at
    // (c + 1) * size - 1, so c runs over [t_begin / size, t_end / size)
    a.c0 = t_begin / p->chunk;
    a.c1 = t_end / p->chunk;
    a.g0 = t_begin / p->group;
    a.g1 = t_end / p->group;
    if (a.c1 < a.c0) a.c1 = a.c0;
    if (a.g1 < a.g0) a.g1 = a.g0;
    a.rope_base = p->rope_base;
    a.groups = gl;
    if (a.c1 == a.c0 && a.g1 == a.g0) return SA_OK;
    return hip_status(sa::launch_summary(a, p->dtype, p->head_dim, s));
  }
  return SA_ERR_INVALID_ARG;
}

int32_t sparse_attn_select(const sa_params* p, const sa_buffers* b, int32_t mode, void* ws,
                           size_t* ws_bytes, void* stream) {
  int32_t st = check_common(p, b);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool append = (mode & SA_SEL_APPEND) != 0;
  mode &= ~SA_SEL_APPEND;
  if (append && mode != SA_SEL_TOPP && mode != SA_SEL_TOPK && mode != SA_SEL_TOPK_BY_SCORE)
    return SA_ERR_INVALID_ARG;
  if (mode == SA_SEL_PYRAMID_TOPK) {
    PyrGeom pg;
    if ((st = pyramid_geom(p, &pg))) return st;
    if (p->q_block < 1 || p->q_block % pg.top_span || p->block_top_k < 1) return SA_ERR_INVALID_ARG;
    // intervals of S blocks whose candidates (about K + S x the entries one
    // block adds) fit the kPsCap slots; none when K leaves too little room
    int64_t per_block = 0;
    for (int l = 0, w = 1; l < p->levels; ++l, w *= p->factor) per_block += p->q_block / w;
    const int64_t room = (int64_t)sa::kPsCap - p->block_top_k - 512;
    const int S = (per_block > 0 && room > 0) ? (int)std::min<int64_t>(room / per_block, 64) : 0;
    const int n_int = (S >= 2) ? (pg.nblk + S - 1) / S : 0;
    const size_t bh = (size_t)p->batch * p->n_q_heads;
    Carver c(ws);
    uint2* prefix = c.take<uint2>(bh);
    uint32_t* tau = c.take<uint32_t>(bh * n_int);
    uint32_t* tau_hi = c.take<uint32_t>(bh * n_int);
    int32_t* cand_len = c.take<int32_t>(bh * n_int);
    uint2* cand = c.take<uint2>(bh * n_int * sa::kPsCap);
    const size_t need = c.size();
    if ((st = workspace_gate(ws, ws_bytes, need))) return st < 0 ? st : SA_OK;
    if (!b->pyr_scores || !b->blk_idx || !b->blk_count) return SA_ERR_INVALID_ARG;
    sa::PyrSelectArgs a{};
    a.prefix = prefix;
    a.S = n_int > 0 ? S : 0;
    a.n_int = n_int;
    a.tau = tau; a.tau_hi = tau_hi; a.cand_len = cand_len; a.cand = cand;
    a.scores = b->pyr_scores; a.blk_idx = b->blk_idx; a.blk_count = b->blk_count;
    a.B = p->batch; a.H = p->n_q_heads; a.N = p->n_ctx; a.levels = p->levels; a.factor = p->factor;
    a.q_block = p->q_block; a.K = p->block_top_k; a.nblk = pg.nblk; a.Nt = pg.Nt;
    {
      int m = p->n_ctx;
      for (int l = 0; l < 8; ++l) {
        a.len[l] = l < p->levels ? m : 0;
        a.soff[l] = l < p->levels ? pg.off[l] : 0;
        if (l < p->levels) m /= p->factor;
      }
    }
    return hip_status(sa::launch_pyramid_select(a, s));
  }
  SelGroups u;
  if ((st = sel_groups(p, &u))) return st;
  if (mode == SA_SEL_TOPP || mode == SA_SEL_TOPK || mode == SA_SEL_TOPK_BY_SCORE) {
    const bool by_score = mode == SA_SEL_TOPK_BY_SCORE;
    if (by_score) mode = SA_SEL_TOPK;
    if (p->r != 16) return SA_ERR_UNSUPPORTED;
    if (by_score && p->top_k > sa::kS2oMax) return SA_ERR_UNSUPPORTED;
    if (mode == SA_SEL_TOPP && (!(p->top_p > 0.f) || std::isnan(p->top_p) || p->min_tokens < 0))
      return SA_ERR_INVALID_ARG;
    if (mode == SA_SEL_TOPK && p->top_k < 1) return SA_ERR_INVALID_ARG;
    GroupList gl = units_of_kind(u, SA_HEAD_RETRIEVAL);
    const int rows = p->batch * gl.n;
    // tokens per workgroup: 2048 (8 per thread), or a larger tile while the
    // rows would need more than two workgroups per compute unit (measured:
    // 1024-token tiles are no faster at 32K and, at more workgroups than the
    // device holds, run the rows in batches).  The workgroups of a row wait
    // for each other, so all of them must be resident together: W stays
    // within the compute units (each holds at least one), which covers 1M
    // tokens.
    const int cus = compute_units();
    const int wmax = std::min(cus, sa::kMaxSelW);
    auto tiles = [&](int per) { return (p->n_ctx + 256 * per - 1) / (256 * per); };
    int per = 8;
    while (per < 16 && ((int64_t)rows * tiles(per) > 2 * cus || tiles(per) > wmax)) per *= 2;
    const int W = tiles(per);
    const int64_t cand_stride = (int64_t)W * 256 * per;
    SelectWs sw = carve_select(nullptr, rows, cand_stride);
    if ((st = workspace_gate(ws, ws_bytes, sw.bytes))) return st < 0 ? st : SA_OK;
    if (gl.n == 0) return SA_OK;
    if (!b->q_idx || !b->k_idx || !b->sel_idx || !b->sel_count) return SA_ERR_INVALID_ARG;
    if (!aligned16(b->k_idx)) return SA_ERR_INVALID_ARG;
    if (W > wmax) return SA_ERR_UNSUPPORTED;
    if (append) {
      if (p->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
      if (!b->k_pre || !b->q_pre || !b->proj_q || !b->proj_k) return SA_ERR_INVALID_ARG;
      if (!aligned16(b->k_pre) || !aligned16(b->q_pre) || !aligned16(b->proj_q) || !aligned16(b->proj_k) ||
          !aligned16(b->q_idx))
        return SA_ERR_INVALID_ARG;
    }
    const bool mass = mode == SA_SEL_TOPP;
    sw = carve_select(ws, rows, cand_stride);
    sa::SelectArgs a{};
    a.q_idx = b->q_idx; a.k_idx = b->k_idx; a.sel_idx = b->sel_idx; a.sel_count = b->sel_count;
    a.B = p->batch; a.Hq = p->n_q_heads; a.Hkv = u.n; a.n = p->n_ctx; a.n_cap = p->n_cap;
    a.G = u.G; a.kv_div = u.kv_div;
    if (mass) {
      a.use_mass = 1;
      a.top_p = p->top_p;
      a.target_count = p->min_tokens;
      a.select_all = (p->top_p >= 1.0f || p->min_tokens >= p->n_ctx) ? 1 : 0;
    } else {
      a.use_mass = 0;
      a.target_count = p->top_k;
      a.select_all = (p->top_k >= p->n_ctx) ? 1 : 0;
    }
    a.W = W;
    a.spin_limit = select_spin_limit();
    const bool fuse = append && !(per > 8 && mass) && u.G <= 16;
    if (append && !fuse) {
      // top-p over 4096-token tiles (registers), or more query heads per row
      // than one projection tile holds: the append as its own launch (the
      // same bits)
      if ((st = sparse_attn_index_build(p, b, SA_IDX_LOWRANK, p->n_ctx - 1, p->n_ctx, stream))) return st;
    }
    a.append = fuse ? 1 : 0;
    a.d = p->head_dim;
    a.k_pre = b->k_pre; a.q_pre = b->q_pre; a.proj_q = b->proj_q; a.proj_k = b->proj_k;
    a.q_idx_w = b->q_idx; a.k_idx_w = b->k_idx;
    a.hist_c = sw.hist_c; a.hist_m = sw.hist_m; a.ctl = sw.ctl; a.slot_a = sw.slot_a; a.slot_b = sw.slot_b;
    a.cand = sw.cand; a.cand_stride = cand_stride;
    a.groups = gl;
    if ((st = hip_status(sa::launch_select_lowrank(a, p->dtype, per, s)))) return st;
    if (!by_score) return SA_OK;
    return hip_status(sa::launch_select_order(a, p->dtype, s));
  }
  if (mode == SA_SEL_ROUTE2_PREFILL) {
    if (p->chunk < 1 || p->group < 1 || p->chunk % p->group) return SA_ERR_INVALID_ARG;
    const int gpc = p->chunk / p->group;
    if (p->top_chunks < 1 || p->top_groups < 1 || p->top_groups > gpc) return SA_ERR_INVALID_ARG;
    if (p->sink_chunks < 0 || p->local_chunks < 0) return SA_ERR_INVALID_ARG;
    if (p->chunk != 128 || p->per_head_sets) return SA_ERR_UNSUPPORTED;   // a query block is one chunk
    if (p->top_chunks > 64 || gpc > 64 || p->top_chunks * p->top_groups > 4096 || p->head_dim > 128)
      return SA_ERR_UNSUPPORTED;
    if (p->n_ctx / p->chunk > 16384) return SA_ERR_UNSUPPORTED;
    // the longest list: sink and local chunks plus the routed groups
    const int64_t longest = ((int64_t)p->sink_chunks + p->local_chunks) * p->chunk +
                            (int64_t)p->top_chunks * p->top_groups * p->group;
    if (p->block_top_k < 1) return SA_ERR_INVALID_ARG;
    if (longest > p->block_top_k) return SA_ERR_CAPACITY;
    GroupList gl = units_of_kind(u, SA_HEAD_ROUTED);
    Carver c(ws);
    c.take<uint32_t>(1);
    if ((st = workspace_gate(ws, ws_bytes, c.size()))) return st < 0 ? st : SA_OK;
    if (gl.n == 0) return SA_OK;
    const int nblk = (p->n_ctx + p->chunk - 1) / p->chunk;
    const bool has_cand = nblk - 1 - p->local_chunks > p->sink_chunks;
    if (!b->q || !b->blk_idx || !b->blk_count) return SA_ERR_INVALID_ARG;
    if (has_cand && (!b->chunk_sum || !b->group_sum)) return SA_ERR_INVALID_ARG;
    if (!aligned16(b->q) || (has_cand && (!aligned16(b->chunk_sum) || !aligned16(b->group_sum))))
      return SA_ERR_INVALID_ARG;
    sa::RouteArgs a{};
    a.q = b->q; a.chunk_sum = b->chunk_sum; a.group_sum = b->group_sum;
    a.B = p->batch; a.Hq = p->n_q_heads; a.Hkv = u.n; a.n = p->n_ctx; a.n_cap = p->n_cap;
    a.G = u.G; a.kv_div = 1; a.chunk = p->chunk; a.group = p->group; a.top_chunks = p->top_chunks;
    a.top_groups = p->top_groups; a.sink_chunks = p->sink_chunks; a.local_chunks = p->local_chunks;
    a.n_cs_cap = p->n_cap / p->chunk; a.n_gs_cap = p->n_cap / p->group;
    a.groups = gl;
    a.prefill = 1; a.nblk = nblk; a.K = p->block_top_k;
    a.blk_idx = b->blk_idx; a.blk_count = b->blk_count;
    return hip_status(sa::launch_route(a, p->dtype, p->head_dim, s));
  }
  if (mode == SA_SEL_ROUTE2) {
    if (p->chunk < 1 || p->group < 1 || p->chunk % p->group) return SA_ERR_INVALID_ARG;
    const int gpc = p->chunk / p->group;
    if (p->top_chunks < 1 || p->top_groups < 1 || p->top_groups > gpc) return SA_ERR_INVALID_ARG;
    if (p->sink_chunks < 0 || p->local_chunks < 0) return SA_ERR_INVALID_ARG;
    if (p->top_chunks > 64 || gpc > 64 || p->top_chunks * p->top_groups > 4096)
      return SA_ERR_UNSUPPORTED;
    if (p->n_ctx / p->chunk > 16384) return SA_ERR_UNSUPPORTED;
    GroupList gl = units_of_kind(u, SA_HEAD_ROUTED);
    Carver c(ws);
    c.take<uint32_t>(1);
    if ((st = workspace_gate(ws, ws_bytes, c.size()))) return st < 0 ? st : SA_OK;
    if (gl.n == 0) return SA_OK;
    // summaries are read only when some complete chunk can be a candidate
    const int kappa = (p->n_ctx - 1) / p->chunk;
    const bool has_cand = kappa - p->local_chunks > p->sink_chunks;
    if (!b->q || !b->sel_idx || !b->sel_count) return SA_ERR_INVALID_ARG;
    if (has_cand && (!b->chunk_sum || !b->group_sum)) return SA_ERR_INVALID_ARG;
    if (!aligned16(b->q) || (has_cand && (!aligned16(b->chunk_sum) || !aligned16(b->group_sum))))
      return SA_ERR_INVALID_ARG;
    sa::RouteArgs a{};
    a.q = b->q; a.chunk_sum = b->chunk_sum; a.group_sum = b->group_sum;
    a.sel_idx = b->sel_idx; a.sel_count = b->sel_count;
    a.B = p->batch; a.Hq = p->n_q_heads; a.Hkv = u.n; a.n = p->n_ctx; a.n_cap = p->n_cap;
    a.G = u.G; a.kv_div = u.kv_div; a.chunk = p->chunk; a.group = p->group; a.top_chunks = p->top_chunks;
    a.top_groups = p->top_groups; a.sink_chunks = p->sink_chunks; a.local_chunks = p->local_chunks;
    a.n_cs_cap = p->n_cap / p->chunk; a.n_gs_cap = p->n_cap / p->group;
    a.groups = gl;
    return hip_status(sa::launch_route(a, p->dtype, p->head_dim, s));
  }
  return SA_ERR_INVALID_ARG;
}

int32_t sparse_attn_decode(const sa_params* p, const sa_buffers* b, void* ws, size_t* ws_bytes,
                           void* stream) {
  return sa::decode_entry(p, b, ws, ws_bytes, stream);
}

int32_t sparse_attn_prefill_chunked(const sa_params* p, const sa_buffers* b, void* ws,
                                    size_t* ws_bytes, void* stream) {
  int32_t st = check_common(p, b);
  if (st) return st;
  PyrGeom pg;
  if ((st = pyramid_geom(p, &pg, true))) return st;
  if (p->q_block < 1 || p->q_block % pg.top_span || p->block_top_k < 1) return SA_ERR_INVALID_ARG;
  if (p->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (p->head_dim != 128 || p->q_block != 128) return SA_ERR_UNSUPPORTED;
  if (p->block_top_k > 8192) return SA_ERR_UNSUPPORTED;   // the selection is staged in LDS
  if (p->n_ctx >= (1 << 23)) return SA_ERR_UNSUPPORTED;   // rows are staged as 32-bit byte offsets
  Carver c(ws);
  c.take<uint32_t>(1);
  if ((st = workspace_gate(ws, ws_bytes, c.size()))) return st < 0 ? st : SA_OK;
  if (!b->q || !b->k_cache || !b->v_cache || !b->blk_idx || !b->blk_count || !b->out)
    return SA_ERR_INVALID_ARG;
  if (p->levels > 1 && (!b->pyr_k || !b->pyr_v)) return SA_ERR_INVALID_ARG;
  sa::PrefillArgs a{};
  a.q = b->q; a.k = b->k_cache; a.v = b->v_cache; a.pk = b->pyr_k; a.pv = b->pyr_v;
  a.blk_idx = b->blk_idx; a.blk_count = b->blk_count; a.out = b->out; a.lse = b->lse;
  a.B = p->batch; a.H = p->n_q_heads; a.N = p->n_ctx; a.Nc = pg.Nc; a.nblk = pg.nblk;
  a.K = p->block_top_k; a.q_block = p->q_block;
  a.Hkv = p->n_kv_heads; a.G = p->n_q_heads / p->n_kv_heads; a.kv_stride = p->n_ctx;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  return hip_status(sa::launch_prefill(a, p->head_dim, static_cast<hipStream_t>(stream)));
}

int32_t sparse_attn_prefill_coarse(const sa_params* p, const sa_buffers* b, void* stream) {
  int32_t st = check_common(p, b);
  if (st) return st;
  PyrGeom pg;
  if ((st = pyramid_geom(p, &pg, false))) return st;
  if (p->q_block < 1 || p->q_block % pg.top_span || p->block_top_k < 1) return SA_ERR_INVALID_ARG;
  if (p->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (p->head_dim != 128 || p->q_block != 128) return SA_ERR_UNSUPPORTED;
  if (p->block_top_k > 8192) return SA_ERR_UNSUPPORTED;
  if (p->n_ctx >= (1 << 23)) return SA_ERR_UNSUPPORTED;
  if (p->levels == 1) return SA_OK;                        // no coarse queries
  if (!b->k_cache || !b->v_cache || !b->blk_idx || !b->blk_count || !b->pyr_q || !b->pyr_k ||
      !b->pyr_v || !b->out_pyr)
    return SA_ERR_INVALID_ARG;
  sa::PrefillArgs a{};
  a.q = b->pyr_q; a.k = b->k_cache; a.v = b->v_cache; a.pk = b->pyr_k; a.pv = b->pyr_v;
  a.blk_idx = b->blk_idx; a.blk_count = b->blk_count; a.out = b->out_pyr; a.lse = nullptr;
  a.B = p->batch; a.H = p->n_q_heads; a.N = p->n_ctx; a.Nc = pg.Nc; a.nblk = pg.nblk;
  a.K = p->block_top_k; a.q_block = p->q_block;
  a.Hkv = p->n_kv_heads; a.G = 1; a.kv_stride = p->n_ctx;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  a.pq = b->pyr_q; a.out_c = b->out_pyr; a.coarse = 1; a.levels = p->levels;
  int span = 1;
  for (int l = 0; l < 8; ++l) {
    a.c_off[l] = (l >= 1 && l < p->levels) ? pg.off[l] - p->n_ctx : 0;
    a.c_span[l] = span;
    if (l + 1 < p->levels) span *= p->factor;
  }
  return hip_status(sa::launch_prefill(a, p->head_dim, static_cast<hipStream_t>(stream)));
}

int32_t sparse_attn_tier_fetch(const sa_params* p, const sa_buffers* b, const sa_tier* t,
                               void* stream) {
  int32_t st = check_common(p, b);
  if (st) return st;
  if (!t) return SA_ERR_INVALID_ARG;
  if (p->per_head_sets) return SA_ERR_UNSUPPORTED;
  SelGroups u;
  if ((st = sel_groups(p, &u))) return st;
  for (int g = 0; g < u.n; ++g)
    if (u.kind[g] != SA_HEAD_ROUTED) return SA_ERR_UNSUPPORTED;
  if (p->chunk < 1 || p->group < 1 || p->chunk % p->group) return SA_ERR_UNSUPPORTED;
  if (p->sink_chunks < 0 || p->local_chunks < 0 || p->top_chunks < 1 || p->top_groups < 1)
    return SA_ERR_INVALID_ARG;
  const int64_t hot_rows = (int64_t)(p->sink_chunks + p->local_chunks + 1) * p->chunk;
  const int64_t max_list = hot_rows + (int64_t)p->top_chunks * p->top_groups * p->group;
  if (max_list > sa::kTierListMax || (int64_t)p->top_chunks * p->top_groups > sa::kTierNeedMax)
    return SA_ERR_UNSUPPORTED;
  if (t->warm_slots < (int64_t)p->top_chunks * p->top_groups || t->warm_slots > sa::kTierSlotsMax)
    return SA_ERR_INVALID_ARG;
  if (!t->cold_k || !t->cold_v || !t->dev_k || !t->dev_v || !t->slot_group || !t->slot_stamp ||
      !t->rows || !b->sel_idx || !b->sel_count)
    return SA_ERR_INVALID_ARG;
  const int64_t dev_rows = hot_rows + (int64_t)t->warm_slots * p->group;
  const int elem = p->dtype == SA_BF16 ? 2 : 4;
  if ((int64_t)p->batch * p->n_kv_heads * p->n_cap * p->head_dim * elem >= (1ll << 62)) return SA_ERR_UNSUPPORTED;
  // the device addresses of the cold store (pinned host memory)
  void* ck = nullptr;
  void* cv = nullptr;
  if (hipHostGetDevicePointer(&ck, const_cast<void*>(t->cold_k), 0) != hipSuccess || !ck ||
      hipHostGetDevicePointer(&cv, const_cast<void*>(t->cold_v), 0) != hipSuccess || !cv) {
    (void)hipGetLastError();
    return SA_ERR_INVALID_ARG;
  }
  sa::TierArgs a{};
  a.sel_idx = b->sel_idx; a.rows = t->rows; a.sel_count = b->sel_count;
  a.cold_k = static_cast<const char*>(ck); a.cold_v = static_cast<const char*>(cv);
  a.dev_k = static_cast<char*>(t->dev_k); a.dev_v = static_cast<char*>(t->dev_v);
  a.slot_group = t->slot_group; a.slot_stamp = t->slot_stamp; a.stats = t->stats;
  a.B = p->batch; a.Hkv = p->n_kv_heads; a.n = p->n_ctx; a.n_cap = p->n_cap;
  a.row_bytes = p->head_dim * elem; a.chunk = p->chunk; a.group = p->group;
  a.sink_chunks = p->sink_chunks; a.local_chunks = p->local_chunks;
  a.warm_slots = t->warm_slots; a.dev_rows = (int32_t)dev_rows; a.step = t->step;
  a.groups = units_of_kind(u, SA_HEAD_ROUTED);
  return hip_status(sa::launch_tier_fetch(a, static_cast<hipStream_t>(stream)));
}

int32_t sparse_attn_prefill_backward(const sa_params* p, const sa_buffers* b, void* ws,
                                     size_t* ws_bytes, void* stream) {
  int32_t st = check_common(p, b);
  if (st) return st;
  if (p->n_q_heads != p->n_kv_heads) return SA_ERR_UNSUPPORTED;
  PyrGeom pg;
  if ((st = pyramid_geom(p, &pg, false))) return st;
  if (p->q_block < 1 || p->q_block % pg.top_span || p->block_top_k < 1) return SA_ERR_INVALID_ARG;
  if (p->dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (p->head_dim != 128 || p->q_block != 128) return SA_ERR_UNSUPPORTED;
  if (p->block_top_k > 8192) return SA_ERR_UNSUPPORTED;
  if (p->n_ctx >= (1 << 23)) return SA_ERR_UNSUPPORTED;
  const int64_t bh = (int64_t)p->batch * p->n_q_heads;
  const int64_t E = pg.Nt;
  // partial rows: one per key, one per (block, chosen entry), and a spare
  const int64_t R = (int64_t)p->n_ctx + (int64_t)pg.nblk * p->block_top_k + 1;
  if (R >= (1ll << 31)) return SA_ERR_UNSUPPORTED;
  Carver c(ws);
  float* delta = c.take<float>(bh * p->n_ctx);
  int32_t* last = c.take<int32_t>(bh * E);
  int32_t* base = c.take<int32_t>(bh * (E + 1));
  uint32_t* err = c.take<uint32_t>(bh);
  float* coarse_k = c.take<float>(bh * pg.Nc * p->head_dim);
  float* coarse_v = c.take<float>(bh * pg.Nc * p->head_dim);
  uint16_t* part_k = c.take<uint16_t>(bh * R * p->head_dim);
  uint16_t* part_v = c.take<uint16_t>(bh * R * p->head_dim);
  if ((st = workspace_gate(ws, ws_bytes, c.size()))) return st < 0 ? st : SA_OK;
  if (!b->q || !b->k_cache || !b->v_cache || !b->blk_idx || !b->blk_count || !b->out ||
      !b->lse || !b->grad_out || !b->grad_q || !b->grad_k || !b->grad_v)
    return SA_ERR_INVALID_ARG;
  if (p->levels > 1 && (!b->pyr_k || !b->pyr_v)) return SA_ERR_INVALID_ARG;
  sa::BwdArgs a{};
  a.q = b->q; a.k = b->k_cache; a.v = b->v_cache; a.pk = b->pyr_k; a.pv = b->pyr_v;
  a.blk_idx = b->blk_idx; a.blk_count = b->blk_count;
  a.out = b->out; a.lse = b->lse; a.dout = b->grad_out;
  a.dq = b->grad_q; a.dk = b->grad_k; a.dv = b->grad_v;
  a.delta = delta; a.last = last; a.base = base; a.err = err;
  a.part_k = part_k; a.part_v = part_v;
  a.coarse_k = coarse_k; a.coarse_v = coarse_v;
  a.R = R;
  a.B = p->batch; a.H = p->n_q_heads; a.N = p->n_ctx; a.Nc = pg.Nc; a.E = (int32_t)E;
  a.nblk = pg.nblk; a.K = p->block_top_k; a.q_block = p->q_block; a.levels = p->levels;
  int span = 1, m = p->n_ctx;
  for (int l = 0; l < 8; ++l) {
    a.off[l] = l < p->levels ? pg.off[l] : 0;
    a.span[l] = span;
    a.cnt[l] = l < p->levels ? m : 0;
    if (l + 1 < p->levels) { span *= p->factor; m /= p->factor; }
  }
  a.scale = (float)(1.0 / std::sqrt((double)p->head_dim));
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  return hip_status(sa::launch_prefill_backward(a, p->head_dim, static_cast<hipStream_t>(stream)));
}

int32_t sparse_attn_prefill_heads(const sa_params* p, const sa_buffers* b, void* stream) {
  int32_t st = check_common(p, b);
  if (st) return st;
  int8_t kinds[sa::kMaxGroups];
  if ((st = group_kinds(p, kinds))) return st;
  if (p->dtype != SA_BF16 || p->head_dim != 128) return SA_ERR_UNSUPPORTED;
  if (p->n_q_heads > sa::kMaxPrefillHeads) return SA_ERR_UNSUPPORTED;
  if (p->n_ctx >= (1 << 23)) return SA_ERR_UNSUPPORTED;   // rows are addressed as 32-bit byte offsets
  const int G = p->n_q_heads / p->n_kv_heads;
  sa::PrefillArgs a{};
  for (int h = 0; h < p->n_q_heads; ++h) {
    const int c = kinds[h / G] == SA_HEAD_LOCAL ? 1 : 0;
    a.cls_heads[c][a.n_cls[c]++] = (uint8_t)h;
  }
  if (a.n_cls[1] > 0 && (p->sinks < 0 || p->window < 0 || (int64_t)p->sinks + p->window < 1))
    return SA_ERR_INVALID_ARG;
  if (!b->q || !b->k_cache || !b->v_cache || !b->out) return SA_ERR_INVALID_ARG;
  if (!aligned16(b->q) || !aligned16(b->k_cache) || !aligned16(b->v_cache) || !aligned16(b->out))
    return SA_ERR_INVALID_ARG;
  a.q = b->q; a.k = b->k_cache; a.v = b->v_cache; a.pk = b->k_cache; a.pv = b->v_cache;
  a.out = b->out;
  a.B = p->batch; a.H = p->n_q_heads; a.N = p->n_ctx; a.Nc = 0;
  a.q_block = 128;                       // queries per workgroup
  a.nblk = (p->n_ctx + a.q_block - 1) / a.q_block;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  a.Hkv = p->n_kv_heads; a.G = G; a.kv_stride = p->n_cap;
  a.sinks = a.n_cls[1] > 0 ? p->sinks : 0;
  a.window = a.n_cls[1] > 0 ? p->window : 0;
  a.units0 = 8 * ((a.B * a.n_cls[0] + 7) / 8) * a.nblk;
  return hip_status(sa::launch_prefill_heads(a, p->head_dim, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
