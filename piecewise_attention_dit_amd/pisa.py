"""ctypes binding of libpisa (C ABI in include/pisa.h).

Argument marshalling only: every step of the hot path runs in the HIP
library.  PyTorch provides device memory and the current stream.  A missing
library raises immediately; there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpisa.so")

PISA_OK, PISA_E_ARG, PISA_E_UNSUPPORTED, PISA_E_WORKSPACE, PISA_E_HIP = range(5)
DTYPES = {"bf16": 0, "f32": 1}
TAYLOR = {"none": 0, "order0": 1, "order1": 2, "hybrid": 3}
DIAG_BYTES = 64


class Params(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("L", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("block", ctypes.c_int32), ("topk", ctypes.c_int32), ("window", ctypes.c_int32),
                ("group", ctypes.c_int32), ("n_cand", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("taylor", ctypes.c_int32), ("scale", ctypes.c_float), ("sink", ctypes.c_int32),
                ("route_lambda", ctypes.c_float)]


class Stats(ctypes.Structure):
    _fields_ = [("qsel", ctypes.c_void_p), ("ksel", ctypes.c_void_p), ("kbar", ctypes.c_void_p),
                ("vsum", ctypes.c_void_p), ("HT", ctypes.c_void_p), ("mcov", ctypes.c_void_p)]


class PisaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Open libpisa.so (built in-tree by piecewise_attention_dit_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m piecewise_attention_dit_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, S, vp, sz = ctypes.POINTER(Params), ctypes.POINTER(Stats), ctypes.c_void_p, ctypes.c_size_t
        L.pisa_validate.argtypes = [P]
        L.pisa_stats_layout.argtypes = [P, ctypes.POINTER(sz)]
        L.pisa_index_layout.argtypes = [P, ctypes.POINTER(sz)]
        L.pisa_workspace_size.argtypes = [P, ctypes.c_int, ctypes.POINTER(sz)]
        L.pisa_block_stats.argtypes = [P, vp, vp, vp, S, vp, sz, vp]
        L.pisa_indexer_topk.argtypes = [P, vp, S, vp, vp, vp, sz, vp]
        L.pisa_sparse_attn_fwd.argtypes = [P, vp, vp, vp, S, vp, vp, vp, vp, sz, vp]
        i32 = ctypes.c_int32
        L.pisa_decode_topk.argtypes = [P, i32, vp, S, vp, vp]
        L.pisa_decode_fwd.argtypes = [P, i32, i32, vp, vp, vp, S, vp, vp, vp, vp, sz, vp]
        L.pisa_decode_fwd_noalloc.argtypes = [P, i32, i32, vp, vp, vp, S, vp, vp, vp, vp]
        L.pisa_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
        L.pisa_probe_hbm_copy.argtypes = [vp, vp, sz, vp]
        L.pisa_probe_hbm_read.argtypes = [vp, sz, vp, vp]
        for f in ("pisa_probe_mfma_bf16", "pisa_probe_hbm_copy", "pisa_probe_hbm_read",
                  "pisa_validate", "pisa_stats_layout", "pisa_index_layout", "pisa_workspace_size",
                  "pisa_block_stats", "pisa_indexer_topk", "pisa_sparse_attn_fwd", "pisa_decode_topk",
                  "pisa_decode_fwd", "pisa_decode_fwd_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        L.pisa_status_string.argtypes = [ctypes.c_int]
        L.pisa_status_string.restype = ctypes.c_char_p
        L.pisa_last_error.restype = ctypes.c_char_p
        L.pisa_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().pisa_status_string(s).decode()
    except Exception:  # library not loadable: plain number
        return f"status {s}"


def _check(status: int):
    if status != PISA_OK:
        raise PisaError(status, lib().pisa_last_error().decode())


def make_params(B, Hq, Hkv, L, d, dtype="bf16", block=64, topk=0, window=0, group=0, n_cand=0,
                causal=False, taylor="order1", scale=0.0, sink=0, route_lambda=0.0) -> Params:
    return Params(B, Hq, Hkv, L, d, DTYPES[dtype] if isinstance(dtype, str) else int(dtype), block,
                  topk, window, group, n_cand, int(bool(causal)),
                  TAYLOR[taylor] if isinstance(taylor, str) else int(taylor), float(scale), int(sink),
                  float(route_lambda))


def validate(p: Params) -> None:
    _check(lib().pisa_validate(ctypes.byref(p)))


def stats_layout(p: Params) -> list[int]:
    arr = (ctypes.c_size_t * 6)()
    _check(lib().pisa_stats_layout(ctypes.byref(p), arr))
    return list(arr)


def index_layout(p: Params) -> list[int]:
    arr = (ctypes.c_size_t * 2)()
    _check(lib().pisa_index_layout(ctypes.byref(p), arr))
    return list(arr)


def workspace_size(p: Params, op: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().pisa_workspace_size(ctypes.byref(p), op, ctypes.byref(n)))
    return n.value


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _tdtype(p: Params):
    return torch.bfloat16 if p.dtype == DTYPES["bf16"] else torch.float32


def alloc_stats(p: Params, device="cuda") -> dict:
    """Caller-owned statistics buffers with the shapes of include/pisa.h."""
    n_blk = -(-p.L // p.block)
    n_sel = -(-p.L // p.group) if p.group >= 1 else n_blk
    td = _tdtype(p)
    st = dict(qsel=torch.empty((p.B, p.Hq, n_sel, p.d), dtype=td, device=device),
              ksel=torch.empty((p.B, p.Hkv, n_blk, p.d), dtype=td, device=device),
              kbar=None, vsum=None, HT=None, mcov=None)
    if p.taylor != TAYLOR["none"]:
        st["kbar"] = torch.empty((p.B, p.Hkv, n_blk, p.d), dtype=torch.float32, device=device)
        st["vsum"] = torch.empty((p.B, p.Hkv, n_blk, p.d), dtype=torch.float32, device=device)
    if p.taylor == TAYLOR["order1"]:
        st["HT"] = torch.empty((p.B, p.Hkv, n_blk, p.d, p.d), dtype=td, device=device)
    elif p.taylor == TAYLOR["hybrid"]:   # the transposed mean first-order matrix (per lo when causal)
        shape = (p.B, p.Hkv, n_blk, p.d, p.d) if p.causal else (p.B, p.Hkv, p.d, p.d)
        st["HT"] = torch.empty(shape, dtype=td, device=device)
    if p.route_lambda > 0:              # covariance norms for routing
        st["mcov"] = torch.empty((p.B, p.Hkv, n_blk), dtype=torch.float32, device=device)
    return st


def _cstats(st: dict) -> Stats:
    return Stats(*(st[k].data_ptr() if st.get(k) is not None else None
                   for k in ("qsel", "ksel", "kbar", "vsum", "HT", "mcov")))


def block_stats(p: Params, q, k, v, stats=None, ws=None, stream=None) -> dict:
    """Stage A.  ws: a device byte buffer of at least workspace_size(p, 0)
    bytes (allocated here when the mode needs one and none is given)."""
    st = stats if stats is not None else alloc_stats(p, q.device)
    cs = _cstats(st)
    need = workspace_size(p, 0)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().pisa_block_stats(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs),
                                  _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))
    return st


def alloc_index(p: Params, device="cuda"):
    n_rows = p.L if p.group >= 1 else -(-p.L // p.block)
    idx = torch.empty((p.B, p.Hq, n_rows, p.topk + p.sink), dtype=torch.int32, device=device)
    cand = None
    if p.group >= 1:
        cand = torch.empty((p.B, p.Hq, -(-p.L // p.group), p.n_cand), dtype=torch.int32, device=device)
    return idx, cand


def indexer_topk(p: Params, q, stats: dict, idx=None, cand=None, want_cand=True, diag=None,
                 stream=None):
    if idx is None:
        idx, c2 = alloc_index(p, q.device)
        if cand is None and want_cand:
            cand = c2
    cs = _cstats(stats)
    ws = _ptr(diag)
    _check(lib().pisa_indexer_topk(ctypes.byref(p), _ptr(q), ctypes.byref(cs), _ptr(idx), _ptr(cand),
                                   ws, DIAG_BYTES if diag is not None else 0, _stream(stream)))
    return idx, cand


def sparse_attn_fwd(p: Params, q, k, v, stats: dict, idx, out=None, lse=None, want_lse=True,
                    ws=None, stream=None):
    """Stage C.  ws: a device byte buffer of at least workspace_size(p, 2)
    bytes (allocated here when the problem needs one and none is given)."""
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((p.B, p.Hq, p.L), dtype=torch.float32, device=q.device)
    need = workspace_size(p, 2)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    cs = _cstats(stats)
    _check(lib().pisa_sparse_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs),
                                      _ptr(idx), _ptr(out), _ptr(lse), _ptr(ws),
                                      ws.numel() if ws is not None else 0, _stream(stream)))
    return out, lse


def decode_topk(p: Params, pos: int, q, stats: dict, idx=None, stream=None):
    """Kept lists [B, Hq, topk + sink] of the new tokens q [B, Hq, d] at
    position pos of the cache the statistics describe."""
    if idx is None:
        idx = torch.empty((p.B, p.Hq, p.topk + p.sink), dtype=torch.int32, device=q.device)
    cs = _cstats(stats)
    _check(lib().pisa_decode_topk(ctypes.byref(p), int(pos), _ptr(q), ctypes.byref(cs), _ptr(idx),
                                  _stream(stream)))
    return idx


def decode_fwd(p: Params, pos: int, q, k, v, stats=None, idx=None, ring: int = 0, out=None, lse=None,
               want_lse=True, ws=None, stream=None):
    """One new token per (b, query head) at position pos: q [B, Hq, d] against
    the cache k, v [B, Hkv, L, d] (or a ring of `ring` slots)."""
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((p.B, p.Hq), dtype=torch.float32, device=q.device)
    need = workspace_size(p, 3)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    cs = _cstats(stats) if stats is not None else None
    _check(lib().pisa_decode_fwd(ctypes.byref(p), int(pos), int(ring), _ptr(q), _ptr(k), _ptr(v),
                                 ctypes.byref(cs) if cs is not None else None, _ptr(idx), _ptr(out), _ptr(lse),
                                 _ptr(ws), ws.numel(), _stream(stream)))
    return out, lse


def decode_fwd_noalloc(p: Params, pos: int, q, k, v, stats=None, idx=None, ring: int = 0, out=None,
                       lse=None, want_lse=True, stream=None):
    """decode_fwd with the split-K partials in the library's fixed scratch
    (no workspace; for callers that cannot allocate).  Allocates out / lse
    here only when they are not given."""
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((p.B, p.Hq), dtype=torch.float32, device=q.device)
    cs = _cstats(stats) if stats is not None else None
    _check(lib().pisa_decode_fwd_noalloc(ctypes.byref(p), int(pos), int(ring), _ptr(q), _ptr(k), _ptr(v),
                                         ctypes.byref(cs) if cs is not None else None, _ptr(idx), _ptr(out),
                                         _ptr(lse), _stream(stream)))
    return out, lse


def probe_mfma_bf16(workgroups: int, iters: int, sink, stream=None) -> float:
    """Roofline probe (include/pisa_roofline.h): enqueue the bf16 MFMA loop;
    returns the dense bf16 FLOPs it executes."""
    _check(lib().pisa_probe_mfma_bf16(int(workgroups), int(iters), _ptr(sink), _stream(stream)))
    return float(workgroups) * 4 * iters * 4 * 32768


def probe_hbm_copy(dst, src, stream=None) -> int:
    """Roofline probe: dst <- src (uint8 tensors of equal size); returns the
    HBM bytes moved (read + write)."""
    n = src.numel() * src.element_size()
    _check(lib().pisa_probe_hbm_copy(_ptr(dst), _ptr(src), n, _stream(stream)))
    return 2 * n


def probe_hbm_read(src, sink, stream=None) -> int:
    """Roofline probe: read every byte of src; returns the bytes read."""
    n = src.numel() * src.element_size()
    _check(lib().pisa_probe_hbm_read(_ptr(src), n, _ptr(sink), _stream(stream)))
    return n


def attention(q, k, v, *, block=64, topk=0, window=0, group=0, n_cand=0, causal=False,
              taylor="order1", scale=0.0, sink=0, route_lambda=0.0, return_all=False):
    """Drop-in forward: (Q, K, V) -> O, running the three library calls."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    dtype = "bf16" if q.dtype == torch.bfloat16 else "f32"
    p = make_params(B, Hq, Hkv, L, d, dtype, block, topk, window, group, n_cand, causal, taylor, scale,
                    sink, route_lambda)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != _tdtype(p):
            raise ValueError(f"{name} must be a contiguous {_tdtype(p)} CUDA tensor")
    st = block_stats(p, q, k, v)
    idx, cand = indexer_topk(p, q, st)
    out, lse = sparse_attn_fwd(p, q, k, v, st, idx)
    if return_all:
        return dict(O=out, lse=lse, idx=idx, cand=cand, stats=st, params=p)
    return out
