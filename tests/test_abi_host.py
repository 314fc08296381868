"""Host-only checks of the C ABI: the library loads, exports every function
include/pisa.h declares, sizes its buffers, and rejects bad arguments before
any launch (no GPU is touched by these tests)."""
import ctypes
import glob
import os
import re

import pytest

from piecewise_attention_dit_amd import pisa
from piecewise_attention_dit_amd import workloads as W

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pisa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(pisa.LIB_PATH), reason="libpisa.so not built")


def _declared():
    names = set()
    for h in sorted(glob.glob(os.path.join(os.path.dirname(HEADER), "*.h"))):
        txt = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(pisa_[a-z0-9_]+)\s*\(", txt))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 16 and "pisa_probe_hbm_read" in names and "pisa_decode_fwd_noalloc" in names
    L = pisa.lib()
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    L = pisa.lib()
    assert L.pisa_abi_version() == 2
    assert L.pisa_status_string(pisa.PISA_E_UNSUPPORTED).decode() == "PISA_E_UNSUPPORTED"


@pytest.mark.parametrize("name", sorted(W.WORKLOADS) + sorted(W.PARITY_CASES))
def test_workloads_validate(name):
    wl = W.get(name)
    p = pisa.make_params(**wl.knobs())
    pisa.validate(p)


def _p(**kw):
    base = dict(B=1, Hq=4, Hkv=2, L=1000, d=128, dtype="bf16", block=64, topk=4, window=0, group=0,
                n_cand=0, causal=False, taylor="order1")
    base.update(kw)
    return pisa.make_params(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), pisa.PISA_E_ARG),
    (dict(Hq=3), pisa.PISA_E_ARG),                       # Hq % Hkv
    (dict(Hq=6, Hkv=2), pisa.PISA_E_UNSUPPORTED),        # ratio 3
    (dict(d=96), pisa.PISA_E_UNSUPPORTED),
    (dict(block=32), pisa.PISA_E_UNSUPPORTED),
    (dict(dtype=7), pisa.PISA_E_ARG),
    (dict(taylor=5), pisa.PISA_E_ARG),
    (dict(sink=-1), pisa.PISA_E_ARG),
    (dict(route_lambda=-1.0), pisa.PISA_E_ARG),
    (dict(route_lambda=float("nan")), pisa.PISA_E_ARG),
    (dict(route_lambda=0.5, taylor="none"), pisa.PISA_E_ARG),
    (dict(route_lambda=0.5, causal=True), pisa.PISA_E_UNSUPPORTED),      # routing is non-causal only
    (dict(route_lambda=0.5, causal=True, group=8, n_cand=8), pisa.PISA_E_UNSUPPORTED),
    (dict(topk=240, sink=25), pisa.PISA_E_UNSUPPORTED),
    (dict(topk=-1), pisa.PISA_E_ARG),
    (dict(topk=257), pisa.PISA_E_UNSUPPORTED),
    (dict(window=64, causal=False), pisa.PISA_E_UNSUPPORTED),
    (dict(group=3, n_cand=8, causal=True), pisa.PISA_E_ARG),    # block % g
    (dict(group=8, n_cand=2, causal=True), pisa.PISA_E_ARG),    # n_cand < topk
    (dict(group=8, n_cand=300, causal=True), pisa.PISA_E_UNSUPPORTED),
    (dict(topk=0, taylor="none", causal=False), pisa.PISA_E_ARG),
    (dict(L=65536 + 64), pisa.PISA_E_UNSUPPORTED),        # more than 1024 blocks
    (dict(scale=float("nan")), pisa.PISA_E_ARG),
])
def test_validation_errors(kw, status):
    with pytest.raises(pisa.PisaError) as ei:
        pisa.validate(_p(**kw))
    assert ei.value.status == status


def test_layouts():
    p = _p(L=1000, group=0)
    n_blk = 16
    sizes = pisa.stats_layout(p)
    assert sizes == [1 * 4 * n_blk * 128 * 2, 1 * 2 * n_blk * 128 * 2, 2 * n_blk * 128 * 4,
                     2 * n_blk * 128 * 4, 2 * n_blk * 128 * 128 * 2, 0]
    assert pisa.index_layout(p) == [1 * 4 * n_blk * 4 * 4, 0]
    assert pisa.index_layout(_p(L=1000, sink=3)) == [1 * 4 * n_blk * (4 + 3) * 4, 0]
    q = _p(L=1000, group=8, n_cand=16, causal=True, dtype="f32")
    sz = pisa.stats_layout(q)
    assert sz[0] == 4 * 125 * 128 * 4 and sz[4] == 2 * n_blk * 128 * 128 * 4
    assert pisa.index_layout(q) == [4 * 1000 * 4 * 4, 4 * 125 * 16 * 4]
    for op in (0, 1, 2):
        assert pisa.workspace_size(p, op) == 0
    # the first-order statistic: per block for order 1, one mean matrix for
    # the hybrid order, none otherwise
    h = _p(L=1000, group=0, taylor="hybrid")
    assert pisa.stats_layout(h)[4] == 2 * 128 * 128 * 2
    # causal rows: one mean per lo (the prefix over the row's candidates)
    hc = _p(L=1000, group=0, taylor="hybrid", causal=True, window=200)
    assert pisa.stats_layout(hc)[4] == 2 * n_blk * 128 * 128 * 2
    assert pisa.workspace_size(hc, 0) == pisa.workspace_size(h, 0)
    assert pisa.stats_layout(h)[2:4] == sizes[2:4]
    for mode in ("none", "order0"):
        assert pisa.stats_layout(_p(L=1000, group=0, taylor=mode, topk=2))[4] == 0
    # the hybrid order's bf16 statistics need fp32 run sums: ceil(16 / 16) runs here
    assert pisa.workspace_size(h, 0) == 1 * 2 * 1 * 128 * 128 * 4
    assert pisa.workspace_size(_p(L=64 * 40, taylor="hybrid"), 0) == 2 * 3 * 128 * 128 * 4
    assert pisa.workspace_size(_p(L=1000, taylor="hybrid", dtype="f32"), 0) == 0
    assert all(pisa.workspace_size(h, op) == 0 for op in (1, 2))
    # routing: covariance norms per block, run sums and an fp32 Hbar copy
    rt = _p(L=1000, route_lambda=0.5)
    assert pisa.stats_layout(rt)[5] == 2 * n_blk * 4 and pisa.stats_layout(p)[5] == 0
    assert pisa.workspace_size(rt, 0) == 2 * 1 * 128 * 128 * 4 + 2 * 128 * 128 * 4
    assert pisa.workspace_size(_p(L=1000, route_lambda=0.5, dtype="f32"), 0) == 2 * 128 * 128 * 4


def test_attention_workspace():
    """PIVOT rows in bf16 without a Taylor tail run key-gathered and need K and
    V^T in MFMA fragment order, 4 B Hkv n_blk block d bytes, when their kept
    sets fit the kernel's LDS (rows x (list + window blocks))."""
    pv = dict(group=8, n_cand=8, causal=True, taylor="none", topk=4)
    assert pisa.workspace_size(_p(L=1000, **pv), 2) == 1 * 2 * 16 * 128 * 64 * 4
    assert pisa.workspace_size(_p(L=1000, block=128, d=64, **pv), 2) == 1 * 2 * 8 * 64 * 128 * 4
    assert pisa.workspace_size(_p(L=1000, **{**pv, "causal": False}), 2) == 1 * 2 * 16 * 128 * 64 * 4
    assert pisa.workspace_size(_p(L=1000, **{**pv, "taylor": "order1"}), 2) == 0
    assert pisa.workspace_size(_p(L=1000, dtype="f32", **pv), 2) == 0
    assert pisa.workspace_size(_p(L=1000, group=0, topk=4, causal=True, taylor="none"), 2) == 0
    # the largest problem the library takes, 1024 blocks, fills the set-up's bitmaps
    assert pisa.workspace_size(_p(L=64 * 1024, **pv), 2) == 1 * 2 * 1024 * 128 * 64 * 4
    with pytest.raises(pisa.PisaError):
        pisa.workspace_size(_p(L=64 * 1025, **pv), 2)
    # a 4096-token window adds 65 blocks per row: past the LDS budget at d 128,
    # within it at d 64
    wide = dict(pv, window=4096, topk=32, n_cand=64)
    assert pisa.workspace_size(_p(L=8192, **wide), 2) == 0
    assert pisa.workspace_size(_p(L=8192, d=64, **wide), 2) == 1 * 2 * 128 * 64 * 64 * 4


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def _call_stats(p, Q=FAKE, K=FAKE, V=FAKE, st=None, ws=None, ws_bytes=0):
    st = st or pisa.Stats(FAKE, FAKE, FAKE, FAKE, FAKE)
    return pisa.lib().pisa_block_stats(ctypes.byref(p), Q, K, V, ctypes.byref(st), ws, ws_bytes, None)


def test_launch_calls_reject_before_launch():
    L = pisa.lib()
    p = _p()
    assert _call_stats(p, Q=None) == pisa.PISA_E_ARG
    assert b"Q is NULL" in L.pisa_last_error()
    assert _call_stats(p, K=FAKE + 4) == pisa.PISA_E_ARG               # misaligned
    assert b"aligned" in L.pisa_last_error()
    assert _call_stats(p, st=pisa.Stats(FAKE, FAKE, None, FAKE, FAKE)) == pisa.PISA_E_ARG
    assert _call_stats(p, ws=None, ws_bytes=128) == pisa.PISA_E_ARG
    hy = _p(taylor="hybrid")                                      # needs a workspace
    assert _call_stats(hy) == pisa.PISA_E_WORKSPACE
    assert _call_stats(hy, ws=FAKE, ws_bytes=pisa.workspace_size(hy, 0) - 16) == pisa.PISA_E_WORKSPACE
    assert _call_stats(hy, ws=FAKE + 4, ws_bytes=pisa.workspace_size(hy, 0)) == pisa.PISA_E_ARG
    rt = _p(route_lambda=0.5)                                     # routing needs mcov
    assert _call_stats(rt, ws=FAKE, ws_bytes=pisa.workspace_size(rt, 0)) == pisa.PISA_E_ARG
    assert b"mcov" in L.pisa_last_error()
    assert _call_stats(_p(d=80)) == pisa.PISA_E_UNSUPPORTED
    assert L.pisa_block_stats(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, 0, None) == pisa.PISA_E_ARG
    st = pisa.Stats(FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.pisa_indexer_topk(ctypes.byref(p), FAKE, ctypes.byref(st), None, None, None, 0,
                               None) == pisa.PISA_E_ARG           # idx NULL with topk > 0
    assert L.pisa_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, ctypes.byref(st), FAKE, None,
                                  None, None, 0, None) == pisa.PISA_E_ARG   # O NULL
    assert L.pisa_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None,
                                  0, None) == pisa.PISA_E_ARG     # stats NULL with Taylor
    assert L.pisa_validate(None) == pisa.PISA_E_ARG
    # decode: causal only, pos inside the cache, ring only for a pure window, workspace
    dc = _p(causal=True, window=128, topk=2)
    ws_need = pisa.workspace_size(dc, 3)
    assert ws_need > 0
    dfwd = lambda pp, pos=5, ring=0, ws=FAKE, wsb=ws_need: L.pisa_decode_fwd(
        ctypes.byref(pp), pos, ring, FAKE, FAKE, FAKE, ctypes.byref(st), FAKE, FAKE, None, ws, wsb, None)
    assert dfwd(_p(causal=False)) == pisa.PISA_E_ARG and b"causal" in L.pisa_last_error()
    assert dfwd(dc, pos=1000) == pisa.PISA_E_ARG and b"pos" in L.pisa_last_error()
    assert dfwd(dc, pos=-1) == pisa.PISA_E_ARG
    assert dfwd(dc, ring=128) == pisa.PISA_E_ARG and b"ring" in L.pisa_last_error()
    assert dfwd(dc, wsb=ws_need - 4) == pisa.PISA_E_WORKSPACE
    assert dfwd(dc, ws=FAKE + 4) == pisa.PISA_E_ARG
    ring_ok = _p(causal=True, window=96, topk=0, taylor="none")
    assert L.pisa_decode_fwd(ctypes.byref(ring_ok), 5, 96, FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                             ws_need, None) == pisa.PISA_E_ARG          # O NULL, after the ring checks pass
    assert b"O is NULL" in L.pisa_last_error()
    assert L.pisa_decode_topk(ctypes.byref(dc), 5, FAKE, ctypes.byref(st), None, None) == pisa.PISA_E_ARG
    # the no-allocation decode: the same checks, and a problem whose partials
    # exceed the library's fixed scratch is refused before any GPU call
    nfwd = lambda pp, pos=5, ring=0: L.pisa_decode_fwd_noalloc(
        ctypes.byref(pp), pos, ring, FAKE, FAKE, FAKE, ctypes.byref(st), FAKE, FAKE, None, None)
    assert nfwd(_p(causal=False)) == pisa.PISA_E_ARG and b"causal" in L.pisa_last_error()
    assert nfwd(dc, pos=1000) == pisa.PISA_E_ARG
    big = _p(B=64, Hq=128, Hkv=128, L=64, causal=True, topk=0, taylor="none")
    assert pisa.workspace_size(big, 3) > 16 << 20
    assert nfwd(big) == pisa.PISA_E_WORKSPACE and b"fixed scratch" in L.pisa_last_error()
