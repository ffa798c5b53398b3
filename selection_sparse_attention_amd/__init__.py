"""Python binding of libsparse_attn (selection-based sparse attention, gfx950).

Argument marshalling only: tensors are passed to the C ABI as raw device
pointers together with torch's current HIP stream; every step of the method
runs inside the library's HIP kernels.  The library must have been built
(``python selection_sparse_attention_amd/build.py``); importing this module
without it raises ImportError - there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparse_attn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python selection_sparse_attention_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

# status codes (sa_status)
SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED = 0, -1, -2
SA_ERR_WORKSPACE, SA_ERR_CAPACITY, SA_ERR_HIP = -3, -4, -5
# enums
SA_BF16, SA_FP32 = 0, 1
HEAD_LOCAL, HEAD_RETRIEVAL, HEAD_ROUTED = 0, 1, 2
IDX_LOWRANK, IDX_CHUNK_SUMMARY, IDX_PYRAMID = 0, 1, 2
SEL_TOPP, SEL_TOPK, SEL_ROUTE2, SEL_PYRAMID_TOPK, SEL_ROUTE2_PREFILL, SEL_TOPK_BY_SCORE = 0, 1, 2, 3, 4, 5
SEL_APPEND = 0x100      # OR'ed into SEL_TOPP / SEL_TOPK / SEL_TOPK_BY_SCORE: fused index append

EXPORTED = ("sparse_attn_index_build", "sparse_attn_select", "sparse_attn_decode",
            "sparse_attn_decode_noalloc", "sparse_attn_prefill_chunked",
            "sparse_attn_prefill_heads", "sparse_attn_prefill_backward",
            "sparse_attn_prefill_coarse", "sparse_attn_tier_fetch",
            "sparse_attn_status_string", "sparse_attn_version")


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_ctx", ctypes.c_int32), ("n_cap", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("head_kind", ctypes.POINTER(ctypes.c_int8)),
        ("rope_base", ctypes.c_float), ("r", ctypes.c_int32),
        ("top_p", ctypes.c_float), ("top_k", ctypes.c_int32),
        ("min_tokens", ctypes.c_int32), ("sinks", ctypes.c_int32),
        ("window", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("group", ctypes.c_int32), ("top_chunks", ctypes.c_int32),
        ("top_groups", ctypes.c_int32), ("sink_chunks", ctypes.c_int32),
        ("local_chunks", ctypes.c_int32), ("levels", ctypes.c_int32),
        ("factor", ctypes.c_int32), ("q_block", ctypes.c_int32),
        ("block_top_k", ctypes.c_int32), ("per_head_sets", ctypes.c_int32),
        ("s2o_tau", ctypes.c_float),
    ]


_BUF_FIELDS = ["q_pre", "k_pre", "q", "k_cache", "v_cache", "proj_q", "proj_k", "q_idx",
               "k_idx", "chunk_sum", "group_sum", "pyr_q", "pyr_k", "pyr_v", "pyr_scores",
               "sel_idx", "sel_count", "blk_idx", "blk_count", "out",
               "grad_out", "lse", "grad_q", "grad_k", "grad_v", "out_pyr"]


class Buffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _BUF_FIELDS]


class Tier(ctypes.Structure):
    """sa_tier: the cold store (pinned host tensors), the device tier and the
    warm slots' tables."""
    _fields_ = [("cold_k", ctypes.c_void_p), ("cold_v", ctypes.c_void_p),
                ("dev_k", ctypes.c_void_p), ("dev_v", ctypes.c_void_p),
                ("warm_slots", ctypes.c_int32), ("step", ctypes.c_int32),
                ("slot_group", ctypes.c_void_p), ("slot_stamp", ctypes.c_void_p),
                ("stats", ctypes.c_void_p), ("rows", ctypes.c_void_p)]


for _name, _args in (
        ("sparse_attn_index_build", [ctypes.POINTER(Params), ctypes.POINTER(Buffers),
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p]),
        ("sparse_attn_select", [ctypes.POINTER(Params), ctypes.POINTER(Buffers), ctypes.c_int32,
                                ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                                ctypes.c_void_p]),
        ("sparse_attn_decode", [ctypes.POINTER(Params), ctypes.POINTER(Buffers),
                                ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                                ctypes.c_void_p]),
        ("sparse_attn_prefill_chunked", [ctypes.POINTER(Params), ctypes.POINTER(Buffers),
                                         ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                                         ctypes.c_void_p]),
        ("sparse_attn_prefill_backward", [ctypes.POINTER(Params), ctypes.POINTER(Buffers),
                                          ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.c_void_p])):
    getattr(_lib, _name).argtypes = _args
    getattr(_lib, _name).restype = ctypes.c_int32
_lib.sparse_attn_decode_noalloc.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Buffers),
                                            ctypes.c_void_p]
_lib.sparse_attn_decode_noalloc.restype = ctypes.c_int32
_lib.sparse_attn_prefill_heads.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Buffers),
                                           ctypes.c_void_p]
_lib.sparse_attn_tier_fetch.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Buffers),
                                        ctypes.POINTER(Tier), ctypes.c_void_p]
_lib.sparse_attn_tier_fetch.restype = ctypes.c_int32
_lib.sparse_attn_prefill_heads.restype = ctypes.c_int32
_lib.sparse_attn_prefill_coarse.argtypes = [ctypes.POINTER(Params), ctypes.POINTER(Buffers),
                                            ctypes.c_void_p]
_lib.sparse_attn_prefill_coarse.restype = ctypes.c_int32
_lib.sparse_attn_status_string.argtypes = [ctypes.c_int32]
_lib.sparse_attn_status_string.restype = ctypes.c_char_p
_lib.sparse_attn_version.restype = ctypes.c_int32


class SparseAttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def status_string(status: int) -> str:
    return _lib.sparse_attn_status_string(int(status)).decode()


def version() -> int:
    return int(_lib.sparse_attn_version())


def make_params(*, batch, n_q_heads, n_kv_heads, head_dim, n_ctx, n_cap=None, dtype="bf16",
                head_kind=None, rope_base=10000.0, r=16, top_p=1.0, top_k=0, min_tokens=0,
                sinks=0, window=0, chunk=64, group=16, top_chunks=16, top_groups=2,
                sink_chunks=4, local_chunks=8, levels=1, factor=4, q_block=128,
                block_top_k=0, per_head_sets=False, s2o_tau=0.0) -> Params:
    """Fill a Params struct.  ``head_kind`` is a per-query-head sequence."""
    p = Params()
    p.batch, p.n_q_heads, p.n_kv_heads, p.head_dim = batch, n_q_heads, n_kv_heads, head_dim
    p.n_ctx = n_ctx
    p.n_cap = n_ctx if n_cap is None else n_cap
    p.dtype = dtype if isinstance(dtype, int) else (SA_BF16 if dtype == "bf16" else SA_FP32)
    kinds = list(head_kind) if head_kind is not None else [HEAD_LOCAL] * n_q_heads
    arr = (ctypes.c_int8 * len(kinds))(*[int(k) for k in kinds])
    p._kinds = arr                                     # keep alive with the struct
    p.head_kind = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int8))
    p.rope_base, p.r, p.top_p, p.top_k, p.min_tokens = rope_base, r, top_p, top_k, min_tokens
    p.sinks, p.window = sinks, window
    p.chunk, p.group, p.top_chunks, p.top_groups = chunk, group, top_chunks, top_groups
    p.sink_chunks, p.local_chunks = sink_chunks, local_chunks
    p.levels, p.factor, p.q_block, p.block_top_k = levels, factor, q_block, block_top_k
    p.per_head_sets = int(per_head_sets)
    p.s2o_tau = float(s2o_tau)
    return p


def params_from_config(cfg, n_cap=None) -> Params:
    """Params for a workloads.DecodeConfig / PrefillConfig-like object."""
    if hasattr(cfg, "n_heads"):     # prefill
        return make_params(batch=cfg.batch, n_q_heads=cfg.n_heads, n_kv_heads=cfg.n_heads,
                           head_dim=cfg.head_dim, n_ctx=cfg.n_ctx, n_cap=n_cap,
                           dtype=cfg.dtype, head_kind=[HEAD_LOCAL] * cfg.n_heads,
                           levels=cfg.levels, factor=cfg.factor, q_block=cfg.q_block,
                           block_top_k=cfg.block_top_k)
    return make_params(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       head_dim=cfg.head_dim, n_ctx=cfg.n_ctx, n_cap=n_cap, dtype=cfg.dtype,
                       head_kind=cfg.head_kind(), rope_base=cfg.rope_base, r=cfg.r,
                       top_p=cfg.top_p, top_k=cfg.top_k, min_tokens=cfg.min_tokens,
                       sinks=cfg.sinks, window=cfg.window, chunk=cfg.chunk, group=cfg.group,
                       top_chunks=cfg.top_chunks, top_groups=cfg.top_groups,
                       sink_chunks=cfg.sink_chunks, local_chunks=cfg.local_chunks,
                       s2o_tau=getattr(cfg, "s2o_tau", 0.0))


def make_buffers(**tensors) -> Buffers:
    """Buffers struct from keyword tensors (or raw ints / None)."""
    b = Buffers()
    for k, v in tensors.items():
        if k not in _BUF_FIELDS:
            raise KeyError(k)
        if v is None:
            continue
        setattr(b, k, v if isinstance(v, int) else v.data_ptr())
    return b


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    return torch.cuda.current_stream().cuda_stream


def _check(status, where):
    if status != SA_OK:
        raise SparseAttnError(status, where)


class Workspace:
    """A reusable device workspace (a zero-filled torch uint8 tensor, grown on
    demand).  Use one per stream.  The library returns the parts it needs zero
    to zero after every call; when the layout changes (batch, head counts or
    head kinds), the buffer is zero-filled again."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None
        self.layout = None

    def get(self, nbytes: int, layout=None) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        elif layout != self.layout:
            self.buf.zero_()
        self.layout = layout
        return self.buf


def _layout(params: Params):
    """What fixes the offsets of a workspace's zero-carrying regions."""
    kinds = (ctypes.string_at(params.head_kind, params.n_q_heads)
             if params.head_kind and params.n_q_heads > 0 else None)
    return (params.batch, params.n_q_heads, params.n_kv_heads, kinds)


_default_ws = {}


def _workspace(ws: Optional[Workspace], fn: str) -> Workspace:
    """The caller's workspace, or a default one per (device, entry point):
    entry points never share a workspace, as their contents persist."""
    if ws is not None:
        return ws
    key = (torch.cuda.current_device(), fn)
    if key not in _default_ws:
        _default_ws[key] = Workspace(f"cuda:{key[0]}")
    return _default_ws[key]


def workspace_size(fn: str, params: Params, bufs: Buffers, mode: int = 0) -> int:
    n = ctypes.c_size_t(0)
    if fn == "select":
        st = _lib.sparse_attn_select(ctypes.byref(params), ctypes.byref(bufs), mode, None,
                                     ctypes.byref(n), None)
    elif fn == "decode":
        st = _lib.sparse_attn_decode(ctypes.byref(params), ctypes.byref(bufs), None,
                                     ctypes.byref(n), None)
    elif fn == "prefill":
        st = _lib.sparse_attn_prefill_chunked(ctypes.byref(params), ctypes.byref(bufs), None,
                                              ctypes.byref(n), None)
    elif fn == "prefill_backward":
        st = _lib.sparse_attn_prefill_backward(ctypes.byref(params), ctypes.byref(bufs), None,
                                               ctypes.byref(n), None)
    else:
        raise ValueError(fn)
    _check(st, f"{fn} (workspace query)")
    return int(n.value)


def index_build(params: Params, bufs: Buffers, mode: int, t_begin: int, t_end: int,
                stream=None):
    _check(_lib.sparse_attn_index_build(ctypes.byref(params), ctypes.byref(bufs), mode,
                                        t_begin, t_end, _stream(stream)), "index_build")


def select(params: Params, bufs: Buffers, mode: int, ws: Optional[Workspace] = None,
           stream=None):
    need = workspace_size("select", params, bufs, mode)
    w = _workspace(ws, "select").get(need, _layout(params))
    n = ctypes.c_size_t(w.numel())
    _check(_lib.sparse_attn_select(ctypes.byref(params), ctypes.byref(bufs), mode,
                                   w.data_ptr(), ctypes.byref(n), _stream(stream)), "select")


def decode(params: Params, bufs: Buffers, ws: Optional[Workspace] = None, stream=None):
    need = workspace_size("decode", params, bufs)
    w = _workspace(ws, "decode").get(need)
    n = ctypes.c_size_t(w.numel())
    _check(_lib.sparse_attn_decode(ctypes.byref(params), ctypes.byref(bufs), w.data_ptr(),
                                   ctypes.byref(n), _stream(stream)), "decode")


def check_selection(sel_count):
    """Raise SparseAttnError when a selection reported failure: a negative
    count among ``sel_count`` (a tensor on any device, holding the counts of
    the rows a selection wrote - slice out groups it does not select for).
    Reading the counts waits for the selection to finish."""
    bad = int((sel_count < 0).sum().item())
    if bad:
        raise SparseAttnError(SA_ERR_HIP, f"select: {bad} row(s) reported a failed selection")


def decode_noalloc(params: Params, bufs: Buffers, stream=None):
    """decode() with the library's static scratch array as its workspace
    (nothing is allocated; concurrent calls on one GPU race)."""
    _check(_lib.sparse_attn_decode_noalloc(ctypes.byref(params), ctypes.byref(bufs),
                                           _stream(stream)), "decode_noalloc")


def prefill_chunked(params: Params, bufs: Buffers, ws: Optional[Workspace] = None,
                    stream=None):
    need = workspace_size("prefill", params, bufs)
    w = _workspace(ws, "prefill").get(need)
    n = ctypes.c_size_t(w.numel())
    _check(_lib.sparse_attn_prefill_chunked(ctypes.byref(params), ctypes.byref(bufs),
                                            w.data_ptr(), ctypes.byref(n), _stream(stream)),
           "prefill_chunked")


def prefill_backward(params: Params, bufs: Buffers, ws: Optional[Workspace] = None,
                     stream=None):
    """Gradients of the pyramid prefill (grad_q, grad_k, grad_v) from
    grad_out, the forward's out and lse, and its lists."""
    need = workspace_size("prefill_backward", params, bufs)
    w = _workspace(ws, "prefill_backward").get(need)
    n = ctypes.c_size_t(w.numel())
    _check(_lib.sparse_attn_prefill_backward(ctypes.byref(params), ctypes.byref(bufs),
                                             w.data_ptr(), ctypes.byref(n), _stream(stream)),
           "prefill_backward")


def make_tier(*, cold_k, cold_v, dev_k, dev_v, slot_group, slot_stamp, rows, step,
              stats=None) -> Tier:
    """Tier struct from tensors (cold_k / cold_v pinned host tensors)."""
    t = Tier()
    t.cold_k, t.cold_v = cold_k.data_ptr(), cold_v.data_ptr()
    t.dev_k, t.dev_v = dev_k.data_ptr(), dev_v.data_ptr()
    t.warm_slots = int(slot_group.shape[-1])
    t.step = int(step)
    t.slot_group, t.slot_stamp = slot_group.data_ptr(), slot_stamp.data_ptr()
    t.stats = stats.data_ptr() if stats is not None else None
    t.rows = rows.data_ptr()
    return t


def tier_fetch(params: Params, bufs: Buffers, tier: Tier, stream=None):
    """Bring the routed groups of this step's lists into the warm slots and
    write the lists as rows of the device tier (tier.rows)."""
    _check(_lib.sparse_attn_tier_fetch(ctypes.byref(params), ctypes.byref(bufs), ctypes.byref(tier),
                                       _stream(stream)), "tier_fetch")


def prefill_coarse(params: Params, bufs: Buffers, stream=None):
    """Coarse queries of the pyramid prefill: every coarse entry of a block
    attends to the block's list and its own level's entries of the block up
    to itself; outputs to bufs.out_pyr (no workspace)."""
    _check(_lib.sparse_attn_prefill_coarse(ctypes.byref(params), ctypes.byref(bufs),
                                           _stream(stream)), "prefill_coarse")


def prefill_heads(params: Params, bufs: Buffers, stream=None):
    """Head-split prefill: local heads over sinks + window, the others
    dense causal (no workspace)."""
    _check(_lib.sparse_attn_prefill_heads(ctypes.byref(params), ctypes.byref(bufs),
                                          _stream(stream)), "prefill_heads")


def raw_call(fn: str, params, bufs, *args):
    """Call an entry point with explicit arguments and return its status
    (used to exercise validation paths)."""
    return int(getattr(_lib, "sparse_attn_" + fn)(params, bufs, *args))
