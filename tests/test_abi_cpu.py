"""The C ABI on a host without a GPU: the library loads, exports every entry
point the header declares, and rejects invalid arguments before launching
anything (every call here fails validation or is a workspace-size query, so
no device pointer is ever dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


def _lib_module():
    from selection_sparse_attention_amd import build as B
    if not os.path.exists(B.library_path()):
        B.build()
    import selection_sparse_attention_amd as sa
    return sa


sa = _lib_module()
FAKE = 0x7F0000000000          # never dereferenced


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int32_t|const char\*)\s+(sparse_attn_\w+)\s*\(", txt,
                                 re.M)))


def test_header_entry_points_are_exported():
    names = declared_functions()
    assert set(names) == set(sa.EXPORTED)
    lib = ctypes.CDLL(sa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    ver = int(re.search(r"#define SPARSE_ATTN_VERSION (\d+)", open(HEADER).read()).group(1))
    assert sa.version() == ver
    assert sa.status_string(0) == "SA_OK"
    assert sa.status_string(-3) == "SA_ERR_WORKSPACE"
    assert sa.status_string(99) == "SA_ERR_UNKNOWN"


def _decode_params(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_ctx=1000, dtype="bf16",
                head_kind=[1] * 4 + [0] * 4, top_p=0.9, min_tokens=8, sinks=4, window=64)
    base.update(kw)
    return sa.make_params(**base)


def _full_bufs():
    names = ["q_pre", "k_pre", "q", "k_cache", "v_cache", "proj_q", "proj_k", "q_idx", "k_idx",
             "chunk_sum", "group_sum", "pyr_q", "pyr_k", "pyr_v", "pyr_scores", "sel_idx",
             "sel_count", "blk_idx", "blk_count", "out"]
    return sa.make_buffers(**{n: FAKE for n in names})


def _select(p, b, mode, ws=None, nbytes=0):
    n = ctypes.c_size_t(nbytes)
    return sa.raw_call("select", ctypes.byref(p), ctypes.byref(b), mode, ws, ctypes.byref(n),
                       None), n.value


def _decode(p, b, ws=None, nbytes=0):
    n = ctypes.c_size_t(nbytes)
    return sa.raw_call("decode", ctypes.byref(p), ctypes.byref(b), ws, ctypes.byref(n),
                       None), n.value


def _index(p, b, mode, t0, t1):
    return sa.raw_call("index_build", ctypes.byref(p), ctypes.byref(b), mode, t0, t1, None)


def test_workspace_queries_return_sizes():
    p, b = _decode_params(), _full_bufs()
    st, n = _select(p, b, sa.SEL_TOPP)
    assert st == sa.SA_OK and n >= 2 * 1 * 1024 * 4          # logits of 2 rows at least
    st, n = _decode(p, b)
    assert st == sa.SA_OK and n >= 2 * 8 * 1 * 130 * 4          # one split per head at least
    pp = sa.make_params(batch=1, n_q_heads=4, n_kv_heads=4, head_dim=128, n_ctx=1024,
                        levels=3, factor=4, q_block=128, block_top_k=64)
    n = ctypes.c_size_t(0)
    assert sa.raw_call("prefill_chunked", ctypes.byref(pp), ctypes.byref(b), None,
                       ctypes.byref(n), None) == sa.SA_OK
    assert n.value >= 256


def test_workspace_too_small_and_misaligned():
    p, b = _decode_params(), _full_bufs()
    _, need = _select(p, b, sa.SEL_TOPP)
    assert _select(p, b, sa.SEL_TOPP, FAKE, need - 1)[0] == sa.SA_ERR_WORKSPACE
    assert _decode(p, b, FAKE, 16)[0] == sa.SA_ERR_WORKSPACE
    assert _select(p, b, sa.SEL_TOPP, FAKE + 8, need)[0] == sa.SA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), sa.SA_ERR_UNSUPPORTED),
    (dict(n_kv_heads=3), sa.SA_ERR_INVALID_ARG),
    (dict(n_cap=999), sa.SA_ERR_INVALID_ARG),
    (dict(batch=0), sa.SA_ERR_INVALID_ARG),
    (dict(dtype=7), sa.SA_ERR_INVALID_ARG),
    (dict(head_kind=[1, 1, 1, 0, 0, 0, 0, 0]), sa.SA_ERR_INVALID_ARG),   # mixed group
    (dict(head_kind=[5] * 8), sa.SA_ERR_INVALID_ARG),
    (dict(top_p=0.0), sa.SA_ERR_INVALID_ARG),
    (dict(top_p=float("nan")), sa.SA_ERR_INVALID_ARG),
    (dict(min_tokens=-1), sa.SA_ERR_INVALID_ARG),
    (dict(r=8), sa.SA_ERR_UNSUPPORTED),
])
def test_select_topp_validation(kw, code):
    assert _select(_decode_params(**kw), _full_bufs(), sa.SEL_TOPP)[0] == code


def test_select_topk_and_route_validation():
    assert _select(_decode_params(top_k=0), _full_bufs(), sa.SEL_TOPK)[0] == sa.SA_ERR_INVALID_ARG
    routed = dict(head_kind=[2] * 8)
    assert _select(_decode_params(top_groups=5, **routed), _full_bufs(),
                   sa.SEL_ROUTE2)[0] == sa.SA_ERR_INVALID_ARG
    assert _select(_decode_params(group=48, **routed), _full_bufs(),
                   sa.SEL_ROUTE2)[0] == sa.SA_ERR_INVALID_ARG
    assert _select(_decode_params(top_chunks=0, **routed), _full_bufs(),
                   sa.SEL_ROUTE2)[0] == sa.SA_ERR_INVALID_ARG
    assert _select(_decode_params(), _full_bufs(), 17)[0] == sa.SA_ERR_INVALID_ARG
    # the routed select's vector loads need 16-byte aligned query and summaries
    p = _decode_params(**routed)
    _, need = _select(p, _full_bufs(), sa.SEL_ROUTE2)
    for name in ("q", "chunk_sum", "group_sum"):
        b = _full_bufs()
        setattr(b, name, FAKE + 8)
        assert _select(p, b, sa.SEL_ROUTE2, FAKE, need)[0] == sa.SA_ERR_INVALID_ARG, name


def test_missing_buffers_are_rejected():
    p = _decode_params()
    _, need = _select(p, _full_bufs(), sa.SEL_TOPP)
    b = _full_bufs()
    b.k_idx = None
    assert _select(p, b, sa.SEL_TOPP, FAKE, need)[0] == sa.SA_ERR_INVALID_ARG
    _, need = _decode(p, _full_bufs())
    b = _full_bufs()
    b.sel_idx = None
    assert _decode(p, b, FAKE, need)[0] == sa.SA_ERR_INVALID_ARG
    b = _full_bufs()
    b.v_cache = None
    assert _decode(p, b, FAKE, need)[0] == sa.SA_ERR_INVALID_ARG


def test_select_append_validation():
    p = _decode_params()
    _, need = _select(p, _full_bufs(), sa.SEL_TOPP | sa.SEL_APPEND)
    assert need > 0
    for mode in (sa.SEL_ROUTE2, sa.SEL_PYRAMID_TOPK, sa.SEL_ROUTE2_PREFILL):
        assert _select(p, _full_bufs(), mode | sa.SEL_APPEND)[0] == sa.SA_ERR_INVALID_ARG
    # fp32 caches: no fused append
    pf = _decode_params(dtype="fp32")
    _, nf = _select(pf, _full_bufs(), sa.SEL_TOPP | sa.SEL_APPEND)
    assert _select(pf, _full_bufs(), sa.SEL_TOPP | sa.SEL_APPEND, FAKE, nf)[0] == \
        sa.SA_ERR_UNSUPPORTED
    # the projection's inputs, present and 16-byte aligned
    for name in ("q_pre", "k_pre", "proj_q", "proj_k"):
        b = _full_bufs()
        setattr(b, name, None)
        assert _select(p, b, sa.SEL_TOPP | sa.SEL_APPEND, FAKE, need)[0] == \
            sa.SA_ERR_INVALID_ARG, name
        b = _full_bufs()
        setattr(b, name, FAKE + 8)
        assert _select(p, b, sa.SEL_TOPP | sa.SEL_APPEND, FAKE, need)[0] == \
            sa.SA_ERR_INVALID_ARG, name


def test_decode_validation():
    b = _full_bufs()
    assert _decode(_decode_params(n_q_heads=6, n_kv_heads=2,
                                  head_kind=[1] * 3 + [0] * 3), b)[0] == sa.SA_ERR_UNSUPPORTED
    assert _decode(_decode_params(sinks=0, window=0), b)[0] == sa.SA_ERR_INVALID_ARG
    assert _decode(_decode_params(sinks=-1), b)[0] == sa.SA_ERR_INVALID_ARG


def test_index_build_validation():
    b = _full_bufs()
    assert _index(_decode_params(), b, sa.IDX_LOWRANK, 5, 5) == sa.SA_ERR_INVALID_ARG
    assert _index(_decode_params(), b, sa.IDX_LOWRANK, -1, 5) == sa.SA_ERR_INVALID_ARG
    assert _index(_decode_params(), b, sa.IDX_LOWRANK, 0, 1001) == sa.SA_ERR_INVALID_ARG
    assert _index(_decode_params(r=32), b, sa.IDX_LOWRANK, 0, 10) == sa.SA_ERR_UNSUPPORTED
    assert _index(_decode_params(), b, 9, 0, 10) == sa.SA_ERR_INVALID_ARG
    assert _index(_decode_params(head_kind=[2] * 8, chunk=60, group=16), b,
                  sa.IDX_CHUNK_SUMMARY, 0, 10) == sa.SA_ERR_INVALID_ARG
    assert _index(_decode_params(head_kind=[2] * 8, rope_base=0.0), b,
                  sa.IDX_CHUNK_SUMMARY, 0, 10) == sa.SA_ERR_INVALID_ARG
    nb = _full_bufs()
    nb.proj_k = None
    assert _index(_decode_params(), nb, sa.IDX_LOWRANK, 0, 10) == sa.SA_ERR_INVALID_ARG


def test_pyramid_validation():
    b = _full_bufs()
    ok = dict(batch=1, n_q_heads=4, n_kv_heads=4, head_dim=128, n_ctx=1024, levels=3, factor=4,
              q_block=128, block_top_k=64)
    mk = lambda **kw: sa.make_params(**{**ok, **kw})
    assert _index(mk(n_ctx=1000), b, sa.IDX_PYRAMID, 0, 1000) == sa.SA_ERR_INVALID_ARG
    assert _index(mk(n_kv_heads=2), b, sa.IDX_PYRAMID, 0, 1024) == sa.SA_ERR_INVALID_ARG
    assert _index(mk(), b, sa.IDX_PYRAMID, 0, 512) == sa.SA_ERR_INVALID_ARG
    assert _index(mk(levels=0), b, sa.IDX_PYRAMID, 0, 1024) == sa.SA_ERR_INVALID_ARG
    assert _index(mk(factor=1), b, sa.IDX_PYRAMID, 0, 1024) == sa.SA_ERR_INVALID_ARG
    assert _select(mk(q_block=100), b, sa.SEL_PYRAMID_TOPK)[0] == sa.SA_ERR_INVALID_ARG
    assert _select(mk(block_top_k=0), b, sa.SEL_PYRAMID_TOPK)[0] == sa.SA_ERR_INVALID_ARG
    n = ctypes.c_size_t(0)
    pf = mk(dtype="fp32")
    assert sa.raw_call("prefill_chunked", ctypes.byref(pf), ctypes.byref(b), None,
                       ctypes.byref(n), None) == sa.SA_ERR_UNSUPPORTED


def test_prefill_limits():
    """The chunked prefill stages a block's selection in LDS and its rows as
    32-bit byte offsets: block_top_k above 8192 and n_ctx of 2^23 or more are
    refused before anything is launched."""
    b = _full_bufs()
    ok = dict(batch=1, n_q_heads=4, n_kv_heads=4, head_dim=128, n_ctx=1024, levels=3, factor=4,
              q_block=128, block_top_k=8192)
    n = ctypes.c_size_t(0)
    pf = sa.make_params(**ok)
    assert sa.raw_call("prefill_chunked", ctypes.byref(pf), ctypes.byref(b), None,
                       ctypes.byref(n), None) == sa.SA_OK
    pf = sa.make_params(**{**ok, "block_top_k": 8193})
    assert sa.raw_call("prefill_chunked", ctypes.byref(pf), ctypes.byref(b), None,
                       ctypes.byref(n), None) == sa.SA_ERR_UNSUPPORTED
    pf = sa.make_params(**{**ok, "head_dim": 64})
    assert sa.raw_call("prefill_chunked", ctypes.byref(pf), ctypes.byref(b), None,
                       ctypes.byref(n), None) == sa.SA_ERR_UNSUPPORTED
    pf = sa.make_params(**{**ok, "n_ctx": (1 << 23) - 256})
    assert sa.raw_call("prefill_chunked", ctypes.byref(pf), ctypes.byref(b), None,
                       ctypes.byref(n), None) == sa.SA_OK
    pf = sa.make_params(**{**ok, "n_ctx": 1 << 23})
    assert sa.raw_call("prefill_chunked", ctypes.byref(pf), ctypes.byref(b), None,
                       ctypes.byref(n), None) == sa.SA_ERR_UNSUPPORTED


def test_decode_noalloc_rejects_a_workspace_larger_than_its_array():
    # fp32 decode of a long context: the split partials need more than the
    # static array holds; the size check runs before any device call
    p = _decode_params(dtype="fp32", batch=8, n_q_heads=32, n_kv_heads=32,
                       head_kind=[1] * 32, n_ctx=200000)
    b = _full_bufs()
    n = ctypes.c_size_t(0)
    assert sa.raw_call("decode", ctypes.byref(p), ctypes.byref(b), None, ctypes.byref(n),
                       None) == sa.SA_OK
    assert n.value > 8 << 20
    st = sa.raw_call("decode_noalloc", ctypes.byref(p), ctypes.byref(b), None)
    assert st == sa.SA_ERR_WORKSPACE


def test_check_selection_flags_negative_counts():
    import torch
    sa.check_selection(torch.tensor([[5, 0], [7, 100]], dtype=torch.int32))
    with pytest.raises(sa.SparseAttnError):
        sa.check_selection(torch.tensor([[5, -1], [7, 100]], dtype=torch.int32))


def test_per_head_sets_validation_and_sizes():
    # the flag is 0 or 1; per-head units need n_q_heads <= 64; a per-head
    # selection has G times the rows (a larger zero-carrying workspace)
    b = _full_bufs()
    st, group_bytes = _select(_decode_params(), b, sa.SEL_TOPP)
    assert st == sa.SA_OK
    st, head_bytes = _select(_decode_params(per_head_sets=True), b, sa.SEL_TOPP)
    assert st == sa.SA_OK and head_bytes > group_bytes
    p = _decode_params()
    p.per_head_sets = 2
    assert _select(p, b, sa.SEL_TOPP)[0] == sa.SA_ERR_INVALID_ARG
    assert _decode(p, b)[0] == sa.SA_ERR_INVALID_ARG
    many = _decode_params(n_q_heads=72, n_kv_heads=8, head_kind=[1] * 72, per_head_sets=True)
    assert _select(many, b, sa.SEL_TOPP)[0] == sa.SA_ERR_UNSUPPORTED
    assert _decode(many, b)[0] == sa.SA_ERR_UNSUPPORTED
    # GQA groups of 3 heads are fine per head (each head is its own unit)
    odd = _decode_params(n_q_heads=6, n_kv_heads=2, head_kind=[1] * 3 + [0] * 3)
    assert _decode(odd, b)[0] == sa.SA_ERR_UNSUPPORTED
    odd.per_head_sets = 1
    assert _decode(odd, b)[0] == sa.SA_OK


def _prefill_heads(p, b):
    return sa.raw_call("prefill_heads", ctypes.byref(p), ctypes.byref(b), None)


def test_prefill_heads_validation():
    b = _full_bufs()
    ok = dict(n_ctx=4096, sinks=4, window=1024)
    assert _prefill_heads(_decode_params(**ok, dtype="fp32"), b) == sa.SA_ERR_UNSUPPORTED
    assert _prefill_heads(_decode_params(**ok, head_dim=64), b) == sa.SA_ERR_UNSUPPORTED
    assert _prefill_heads(_decode_params(n_ctx=1 << 23, sinks=4, window=8), b) == \
        sa.SA_ERR_UNSUPPORTED
    assert _prefill_heads(_decode_params(n_ctx=4096, sinks=0, window=0), b) == \
        sa.SA_ERR_INVALID_ARG
    assert _prefill_heads(_decode_params(n_ctx=4096, sinks=-1, window=8), b) == \
        sa.SA_ERR_INVALID_ARG
    # labels must agree inside a GQA group
    mixed = _decode_params(**ok, head_kind=[1, 0, 1, 1, 0, 0, 0, 0])
    assert _prefill_heads(mixed, b) == sa.SA_ERR_INVALID_ARG
    # a missing or misaligned buffer
    nb = _full_bufs()
    nb.out = None
    assert _prefill_heads(_decode_params(**ok), nb) == sa.SA_ERR_INVALID_ARG
    mb = _full_bufs()
    mb.q = FAKE + 8
    assert _prefill_heads(_decode_params(**ok), mb) == sa.SA_ERR_INVALID_ARG


def test_route_prefill_validation():
    b = _full_bufs()
    base = dict(n_ctx=128 * 40, head_kind=[2] * 8, chunk=128, group=32, top_chunks=4,
                top_groups=2, sink_chunks=2, local_chunks=3, levels=1, q_block=128)
    need = (2 + 3) * 128 + 4 * 2 * 32
    st, _ = _select(_decode_params(**base, block_top_k=need), b, sa.SEL_ROUTE2_PREFILL)
    assert st == sa.SA_OK
    assert _select(_decode_params(**base, block_top_k=need - 1), b,
                   sa.SEL_ROUTE2_PREFILL)[0] == sa.SA_ERR_CAPACITY
    bad_chunk = dict(base, chunk=64, group=16)
    assert _select(_decode_params(**bad_chunk, block_top_k=need), b,
                   sa.SEL_ROUTE2_PREFILL)[0] == sa.SA_ERR_UNSUPPORTED
    assert _select(_decode_params(**base, block_top_k=need, per_head_sets=True), b,
                   sa.SEL_ROUTE2_PREFILL)[0] == sa.SA_ERR_UNSUPPORTED
    # a GQA prefill over lists is allowed with one level only
    n = ctypes.c_size_t(0)
    p1 = _decode_params(**base, block_top_k=need)
    assert sa.raw_call("prefill_chunked", ctypes.byref(p1), ctypes.byref(b), None,
                       ctypes.byref(n), None) == sa.SA_OK
    p3 = _decode_params(**dict(base, levels=3, factor=4), block_top_k=need)
    assert sa.raw_call("prefill_chunked", ctypes.byref(p3), ctypes.byref(b), None,
                       ctypes.byref(n), None) == sa.SA_ERR_INVALID_ARG


def test_s2o_validation():
    b = _full_bufs()
    topk = dict(top_k=4096)
    assert _select(_decode_params(**topk), b, sa.SEL_TOPK_BY_SCORE)[0] == sa.SA_OK
    assert _select(_decode_params(top_k=8193), b, sa.SEL_TOPK_BY_SCORE)[0] == sa.SA_ERR_UNSUPPORTED
    assert _decode(_decode_params(s2o_tau=0.01), b)[0] == sa.SA_OK
    assert _decode(_decode_params(s2o_tau=-1.0), b)[0] == sa.SA_ERR_INVALID_ARG
    assert _decode(_decode_params(s2o_tau=float("nan")), b)[0] == sa.SA_ERR_INVALID_ARG
    assert _decode(_decode_params(s2o_tau=0.01, dtype="fp32"), b)[0] == sa.SA_ERR_UNSUPPORTED
    # the first pass needs sinks or a window
    assert _decode(_decode_params(s2o_tau=0.01, sinks=0, window=0, head_kind=[1] * 8), b)[0] == \
        sa.SA_ERR_INVALID_ARG


def test_prefill_backward_validation_and_size():
    """The backward pass: its workspace holds, per head, the per-entry
    tables and one bf16 partial row of dK and of dV per (block, chosen
    entry) and per level-0 key; grouped heads, fp32, d = 64 and a missing
    gradient buffer are refused before anything is launched."""
    b = _full_bufs()
    for name in ("grad_out", "lse", "grad_q", "grad_k", "grad_v"):
        setattr(b, name, FAKE)
    ok = dict(batch=2, n_q_heads=4, n_kv_heads=4, head_dim=128, n_ctx=1024, levels=3, factor=4,
              q_block=128, block_top_k=300)
    n = ctypes.c_size_t(0)
    pf = sa.make_params(**ok)
    assert sa.raw_call("prefill_backward", ctypes.byref(pf), ctypes.byref(b), None,
                       ctypes.byref(n), None) == sa.SA_OK
    bh, N, E, nblk = 2 * 4, 1024, 1024 + 256 + 64, 8
    R = N + nblk * 300
    assert n.value >= bh * R * 128 * 2 * 2 + bh * (256 + 64) * 128 * 4 * 2
    assert n.value <= bh * R * 128 * 2 * 2 + bh * (256 + 64) * 128 * 4 * 2 + bh * (N + 2 * E + 2) * 4 + 64 * 1024
    for kw, code in ((dict(n_kv_heads=2), sa.SA_ERR_UNSUPPORTED),
                     (dict(dtype="fp32"), sa.SA_ERR_UNSUPPORTED),
                     (dict(head_dim=64), sa.SA_ERR_UNSUPPORTED),
                     (dict(block_top_k=8193), sa.SA_ERR_UNSUPPORTED),
                     (dict(n_ctx=1000), sa.SA_ERR_INVALID_ARG)):       # not a multiple of p^(L-1)
        pf = sa.make_params(**{**ok, **kw})
        assert sa.raw_call("prefill_backward", ctypes.byref(pf), ctypes.byref(b), None,
                           ctypes.byref(n), None) == code, kw
    pf = sa.make_params(**ok)
    n = ctypes.c_size_t(1 << 40)
    for name in ("grad_out", "lse", "grad_q", "grad_k", "grad_v"):
        setattr(b, name, None)
        assert sa.raw_call("prefill_backward", ctypes.byref(pf), ctypes.byref(b), FAKE,
                           ctypes.byref(n), None) == sa.SA_ERR_INVALID_ARG, name
        setattr(b, name, FAKE)


def test_prefill_coarse_validation():
    """The coarse-query prefill: one level means no coarse queries (SA_OK,
    nothing launched); grouped heads, fp32, d = 64, a list longer than 8192,
    a length the top span does not divide and a missing coarse buffer are
    refused before anything is launched."""
    b = _full_bufs()
    b.out_pyr = FAKE
    ok = dict(batch=2, n_q_heads=4, n_kv_heads=4, head_dim=128, n_ctx=1024, levels=3, factor=4,
              q_block=128, block_top_k=300)
    pf = sa.make_params(**{**ok, "levels": 1})
    assert sa.raw_call("prefill_coarse", ctypes.byref(pf), ctypes.byref(b), None) == sa.SA_OK
    for kw, code in ((dict(n_kv_heads=2), sa.SA_ERR_INVALID_ARG),
                     (dict(dtype="fp32"), sa.SA_ERR_UNSUPPORTED),
                     (dict(head_dim=64), sa.SA_ERR_UNSUPPORTED),
                     (dict(block_top_k=8193), sa.SA_ERR_UNSUPPORTED),
                     (dict(q_block=64), sa.SA_ERR_UNSUPPORTED),
                     (dict(n_ctx=1000), sa.SA_ERR_INVALID_ARG)):
        pf = sa.make_params(**{**ok, **kw})
        assert sa.raw_call("prefill_coarse", ctypes.byref(pf), ctypes.byref(b), None) == code, kw
    pf = sa.make_params(**ok)
    for name in ("pyr_q", "pyr_k", "pyr_v", "out_pyr", "blk_idx", "blk_count"):
        keep = getattr(b, name)
        setattr(b, name, None)
        assert sa.raw_call("prefill_coarse", ctypes.byref(pf), ctypes.byref(b), None) == \
            sa.SA_ERR_INVALID_ARG, name
        setattr(b, name, keep)


def test_tier_fetch_validation():
    """The tier fetch refuses, before anything runs: heads that are not all
    routed, per-head sets, a chunk that groups do not divide, fewer warm
    slots than one step routes (or more than 4096), lists longer than 8192,
    and missing tables or stores."""
    b = _full_bufs()
    ok = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, n_ctx=4096,
              head_kind=[sa.HEAD_ROUTED] * 8, chunk=64, group=16, top_chunks=4, top_groups=2,
              sink_chunks=2, local_chunks=3)

    def tier(**kw):
        t = sa.Tier()
        t.cold_k = t.cold_v = t.dev_k = t.dev_v = FAKE
        t.slot_group = t.slot_stamp = t.rows = FAKE
        t.warm_slots, t.step = 8, 1
        for k, v in kw.items():
            setattr(t, k, v)
        return t

    def call(pkw, **tkw):
        p = sa.make_params(**{**ok, **pkw})
        return sa.raw_call("tier_fetch", ctypes.byref(p), ctypes.byref(b), ctypes.byref(tier(**tkw)), None)

    assert call({"head_kind": [sa.HEAD_ROUTED] * 4 + [sa.HEAD_LOCAL] * 4}) == sa.SA_ERR_UNSUPPORTED
    assert call({"per_head_sets": True}) == sa.SA_ERR_UNSUPPORTED
    assert call({"chunk": 64, "group": 24}) == sa.SA_ERR_UNSUPPORTED
    assert call({}, warm_slots=7) == sa.SA_ERR_INVALID_ARG
    assert call({}, warm_slots=4097) == sa.SA_ERR_INVALID_ARG
    assert call({"top_chunks": 64, "top_groups": 4, "sink_chunks": 64}) == sa.SA_ERR_UNSUPPORTED
    assert call({}, slot_group=None) == sa.SA_ERR_INVALID_ARG
    assert call({}, cold_v=None) == sa.SA_ERR_INVALID_ARG
    assert call({}, rows=None) == sa.SA_ERR_INVALID_ARG
