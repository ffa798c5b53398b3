// C ABI of the sparse attention library: argument validation, workspace
// sizing and carving, and kernel launch on the caller's stream.  Nothing here
// allocates, frees, copies to the host or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/sparse_attn.h"
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

int32_t pyramid_geom(const sa_params* p, PyrGeom* g) {
  if (p->levels < 1 || p->levels > 8 || p->factor < 2) return SA_ERR_INVALID_ARG;
  if (p->n_q_heads != p->n_kv_heads) return SA_ERR_INVALID_ARG;
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
constexpr int kSelTile = 1024;

struct SelectWs {
  float* logits; uint32_t* cnt1; double* mass1; uint32_t* maxkey; sa::RowState* state;
  uint64_t* lookback;
  int tiles; int64_t row_stride; size_t bytes;
};

// The regions that must be zero when a call starts (the level-1 histogram and
// the row maxima, returned to zero by every call) come first, so their
// offsets depend on the number of rows only, not on n_ctx.
SelectWs carve_select(void* ws, int rows, int n) {
  SelectWs s{};
  s.tiles = (n + kSelTile - 1) / kSelTile;
  s.row_stride = (int64_t)s.tiles * kSelTile;
  Carver c(ws);
  s.cnt1 = c.take<uint32_t>((size_t)rows * 4096);
  s.mass1 = c.take<double>((size_t)rows * 4096);
  s.maxkey = c.take<uint32_t>((size_t)rows);
  s.state = c.take<sa::RowState>((size_t)rows);
  s.lookback = c.take<uint64_t>((size_t)rows * s.tiles);
  s.logits = c.take<float>((size_t)rows * s.row_stride);
  s.bytes = c.size();
  return s;
}

// ---------------------------------------------------------------- decode ws
constexpr int kDecodeTps = 256;           // fp32 caches: list entries per split
constexpr int kDecodeMinChunk = 64;       // bf16 caches: smallest work item (list entries)
constexpr int kMaxDecodeItems = 8192;     // bf16 caches: work items one launch may hold
constexpr int kMaxDecodeSplits = 8192;     // contexts up to 2M tokens

// Compute units of the current device (queried once per device).
int compute_units() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cache[dev] = n;
  return n;
}

int decode_max_count(const sa_params* p, const int8_t* kinds) {
  int mc = 0;
  for (int g = 0; g < p->n_kv_heads; ++g) {
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
  const int G = p->n_q_heads / p->n_kv_heads;
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
  int8_t kinds[sa::kMaxGroups];
  if ((st = group_kinds(p, kinds))) return st;
  if (mode == SA_SEL_TOPP || mode == SA_SEL_TOPK) {
    if (p->r != 16) return SA_ERR_UNSUPPORTED;
    if (mode == SA_SEL_TOPP && (!(p->top_p > 0.f) || std::isnan(p->top_p) || p->min_tokens < 0))
      return SA_ERR_INVALID_ARG;
    if (mode == SA_SEL_TOPK && p->top_k < 1) return SA_ERR_INVALID_ARG;
    GroupList gl = groups_of_kind(p, kinds, SA_HEAD_RETRIEVAL);
    const int rows = p->batch * gl.n;
    SelectWs sw = carve_select(nullptr, rows, p->n_ctx);
    if ((st = workspace_gate(ws, ws_bytes, sw.bytes))) return st < 0 ? st : SA_OK;
    if (gl.n == 0) return SA_OK;
    if (!b->q_idx || !b->k_idx || !b->sel_idx || !b->sel_count) return SA_ERR_INVALID_ARG;
    if (!aligned16(b->k_idx)) return SA_ERR_INVALID_ARG;
    sw = carve_select(ws, rows, p->n_ctx);
    sa::SelectArgs a{};
    a.q_idx = b->q_idx; a.k_idx = b->k_idx; a.sel_idx = b->sel_idx; a.sel_count = b->sel_count;
    a.B = p->batch; a.Hq = p->n_q_heads; a.Hkv = p->n_kv_heads; a.n = p->n_ctx; a.n_cap = p->n_cap;
    a.G = G;
    if (mode == SA_SEL_TOPP) {
      a.use_mass = 1;
      a.top_p = p->top_p;
      a.target_count = p->min_tokens;
      a.select_all = (p->top_p >= 1.0f || p->min_tokens >= p->n_ctx) ? 1 : 0;
    } else {
      a.use_mass = 0;
      a.target_count = p->top_k;
      a.select_all = (p->top_k >= p->n_ctx) ? 1 : 0;
    }
    a.tiles = sw.tiles; a.row_stride = sw.row_stride;
    a.logits = sw.logits; a.cnt1 = sw.cnt1; a.mass1 = sw.mass1; a.maxkey = sw.maxkey;
    a.state = sw.state;
    a.lookback = sw.lookback; a.groups = gl;
    return hip_status(sa::launch_select_lowrank(a, p->dtype, s));
  }
  if (mode == SA_SEL_ROUTE2) {
    if (p->chunk < 1 || p->group < 1 || p->chunk % p->group) return SA_ERR_INVALID_ARG;
    const int gpc = p->chunk / p->group;
    if (p->top_chunks < 1 || p->top_groups < 1 || p->top_groups > gpc) return SA_ERR_INVALID_ARG;
    if (p->sink_chunks < 0 || p->local_chunks < 0) return SA_ERR_INVALID_ARG;
    if (p->top_chunks > 64 || gpc > 64 || p->top_chunks * p->top_groups > 4096)
      return SA_ERR_UNSUPPORTED;
    if (p->n_ctx / p->chunk > 16384) return SA_ERR_UNSUPPORTED;
    GroupList gl = groups_of_kind(p, kinds, SA_HEAD_ROUTED);
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
    a.B = p->batch; a.Hq = p->n_q_heads; a.Hkv = p->n_kv_heads; a.n = p->n_ctx; a.n_cap = p->n_cap;
    a.G = G; a.chunk = p->chunk; a.group = p->group; a.top_chunks = p->top_chunks;
    a.top_groups = p->top_groups; a.sink_chunks = p->sink_chunks; a.local_chunks = p->local_chunks;
    a.n_cs_cap = p->n_cap / p->chunk; a.n_gs_cap = p->n_cap / p->group;
    a.groups = gl;
    return hip_status(sa::launch_route(a, p->dtype, p->head_dim, s));
  }
  return SA_ERR_INVALID_ARG;
}

int32_t sparse_attn_decode(const sa_params* p, const sa_buffers* b, void* ws, size_t* ws_bytes,
                           void* stream) {
  int32_t st = check_common(p, b);
  if (st) return st;
  int8_t kinds[sa::kMaxGroups];
  if ((st = group_kinds(p, kinds))) return st;
  const int G = p->n_q_heads / p->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return SA_ERR_UNSUPPORTED;
  bool any_local = false, any_list = false;
  uint64_t local_mask = 0;
  for (int g = 0; g < p->n_kv_heads; ++g) {
    if (kinds[g] == SA_HEAD_LOCAL) { any_local = true; local_mask |= 1ull << g; }
    else any_list = true;
  }
  if (any_local && (p->sinks < 0 || p->window < 0 || (int64_t)p->sinks + p->window < 1))
    return SA_ERR_INVALID_ARG;
  int tps = kDecodeTps, max_splits, target_items = 0;
  size_t n_partial;
  if (p->dtype == SA_BF16) {
    // work items: the step's visible tokens spread over one item per
    // workgroup slot (two per compute unit, one for 8-head groups, whose
    // workgroups use a whole unit's registers); the plan itself is made on
    // the device
    const int groups = p->batch * p->n_kv_heads;
    target_items = (G > 4 ? 1 : 2) * compute_units();
    max_splits = target_items + groups;        // bound on the item count
    if (max_splits > kMaxDecodeItems) return SA_ERR_UNSUPPORTED;
    n_partial = (size_t)max_splits * G * (p->head_dim + 2);
  } else {
    const int max_count = decode_max_count(p, kinds);
    max_splits = (max_count + tps - 1) / tps;
    if (max_splits > kMaxDecodeSplits) return SA_ERR_UNSUPPORTED;
    n_partial = (size_t)p->batch * p->n_q_heads * max_splits * (p->head_dim + 2);
  }
  Carver c(ws);
  float* partial = c.take<float>(n_partial);
  int2* plan = (p->dtype == SA_BF16) ? c.take<int2>((size_t)p->batch * p->n_kv_heads) : nullptr;
  if ((st = workspace_gate(ws, ws_bytes, c.size()))) return st < 0 ? st : SA_OK;
  if (!b->q || !b->k_cache || !b->v_cache || !b->out) return SA_ERR_INVALID_ARG;
  if (any_list && (!b->sel_idx || !b->sel_count)) return SA_ERR_INVALID_ARG;
  if (!aligned16(b->q) || !aligned16(b->k_cache) || !aligned16(b->v_cache)) return SA_ERR_INVALID_ARG;
  sa::DecodeArgs a{};
  a.q = b->q; a.k = b->k_cache; a.v = b->v_cache; a.sel_idx = b->sel_idx; a.sel_count = b->sel_count;
  a.out = b->out; a.partial = partial;
  a.B = p->batch; a.Hq = p->n_q_heads; a.Hkv = p->n_kv_heads; a.n = p->n_ctx; a.n_cap = p->n_cap;
  a.G = G; a.sinks = p->sinks; a.window = p->window; a.tps = tps; a.max_splits = max_splits;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  a.local_mask = local_mask;
  a.target_items = target_items;
  a.min_chunk = kDecodeMinChunk;
  a.plan = plan;
  return hip_status(sa::launch_decode(a, p->dtype, p->head_dim, static_cast<hipStream_t>(stream)));
}

int32_t sparse_attn_prefill_chunked(const sa_params* p, const sa_buffers* b, void* ws,
                                    size_t* ws_bytes, void* stream) {
  int32_t st = check_common(p, b);
  if (st) return st;
  PyrGeom pg;
  if ((st = pyramid_geom(p, &pg))) return st;
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
  a.blk_idx = b->blk_idx; a.blk_count = b->blk_count; a.out = b->out;
  a.B = p->batch; a.H = p->n_q_heads; a.N = p->n_ctx; a.Nc = pg.Nc; a.nblk = pg.nblk;
  a.K = p->block_top_k; a.q_block = p->q_block;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)p->head_dim));
  return hip_status(sa::launch_prefill(a, p->head_dim, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
