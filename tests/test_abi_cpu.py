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
