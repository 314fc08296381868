"""GPU parity of the decode path (one new token per (batch, query head)):
pisa_decode_topk against the oracle's decode selection (bit-exact), and
pisa_decode_fwd against the oracle's decode step, with the lists it selects,
with lists reused from another query (another layer's selection), from a
cache whose slots past the token hold unrelated values (a decoder has not
filled them), and from a ring buffer.  Bar: lists bit-exact; outputs within
max-abs 2e-2 / mean-abs 2e-3 (bf16) or 1e-4 (fp32), lse within 1e-2 / 1e-5."""
import numpy as np
import pytest
import torch

from gpu_common import TOL, problem
from oracle import pisa_oracle as po
from piecewise_attention_dit_amd import pisa
from piecewise_attention_dit_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    dict(B=1, Hq=4, Hkv=2, L=1000, d=128, dtype="bf16", block=64, topk=3, window=200, taylor="order1"),
    dict(B=2, Hq=2, Hkv=1, L=900, d=64, dtype="bf16", block=128, topk=2, window=0, taylor="hybrid", sink=1),
    dict(B=1, Hq=8, Hkv=1, L=1100, d=128, dtype="bf16", block=64, topk=4, window=300, taylor="order0"),
    dict(B=1, Hq=2, Hkv=2, L=700, d=128, dtype="bf16", block=128, topk=2, window=150, taylor="none", sink=2),
    dict(B=1, Hq=2, Hkv=1, L=600, d=64, dtype="f32", block=64, topk=2, window=100, taylor="order1"),
    dict(B=1, Hq=4, Hkv=2, L=1300, d=128, dtype="bf16", block=64, topk=3, window=256, taylor="hybrid"),
    # B * Hkv = 32 (kv groups): 16 split-K workgroups each, fewer than the cap
    dict(B=4, Hq=32, Hkv=8, L=640, d=128, dtype="bf16", block=64, topk=2, window=128, taylor="order1"),
    dict(B=1, Hq=2, Hkv=2, L=500, d=64, dtype="f32", block=64, topk=1, window=70, taylor="hybrid"),
]


def _inputs(kn, seed):
    wl = W.Workload("decode", recipe="gauss", **dict(kn, causal=True))
    return W.make_inputs(wl, seed=seed)


def _check(out, lse, o_ref, l_ref, tol, what):
    o = out.cpu().double().numpy()
    assert np.isfinite(o).all(), what
    d = np.abs(o - o_ref)
    assert d.max() <= tol["max_abs"], f"{what}: max abs error {d.max()}"
    assert d.mean() <= tol["mean_abs"], f"{what}: mean abs error {d.mean()}"
    assert np.abs(lse.cpu().double().numpy() - l_ref).max() <= tol["lse"], f"{what}: lse"


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_decode_matches_oracle(ci):
    kn = dict(CASES[ci], causal=True)
    P = problem(kn)
    q, k, v = _inputs(kn, 11 + ci)
    qa, ka, va = (x.double().numpy() for x in (q, k, v))
    st_ref = po.block_stats(qa, ka, va, P)
    p = pisa.make_params(**kn)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    st = pisa.block_stats(p, dq, dk, dv)
    tol = TOL[P.dtype]
    L, bs = P.L, P.block
    print(f"[decode] case {ci}: {kn} splits workspace {pisa.workspace_size(p, 3)} B", flush=True)
    for pos in (0, bs - 1, bs, L // 2 + 3, L - 1):
        print(f"[decode] case {ci} pos {pos}", flush=True)
        qt = dq[:, :, pos].contiguous()
        idx = pisa.decode_topk(p, pos, qt, st)
        ref_idx = po.decode_select(qa[:, :, pos], st_ref, P, pos)
        assert np.array_equal(idx.cpu().numpy().astype(np.int64), ref_idx), (pos, idx.cpu(), ref_idx)
        # the lists of another query (a reused selection)
        other = (pos * 7 + 5) % L
        idx_o = pisa.decode_topk(p, pos, dq[:, :, other].contiguous(), st)
        ref_o = po.decode_select(qa[:, :, other], st_ref, P, pos)
        assert np.array_equal(idx_o.cpu().numpy().astype(np.int64), ref_o)
        for lists, ref_lists in ((idx, ref_idx), (idx_o, ref_o)):
            out, lse = pisa.decode_fwd(p, pos, qt, dk, dv, st, lists)
            torch.cuda.synchronize()
            o_ref, l_ref = po.decode_attend(qa[:, :, pos], ka, va, st_ref, ref_lists, P, pos)
            _check(out, lse, o_ref, l_ref, tol, f"pos {pos}")


@pytest.mark.parametrize("ci", [0, 1, 5, 6, 7])
def test_decode_unfilled_cache(ci):
    """A decoder at position pos has filled slots 0 .. pos only: the slots
    after pos hold unrelated finite values here, and the statistics are taken
    over that cache.  The step must match the oracle on that cache and equal,
    bit for bit, the step on the cache the sequence itself fills."""
    kn = dict(CASES[ci], causal=True)
    P = problem(kn)
    q, k, v = _inputs(kn, 41 + ci)
    p = pisa.make_params(**kn)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    st = pisa.block_stats(p, dq, dk, dv)
    tol = TOL[P.dtype]
    g = torch.Generator().manual_seed(77 + ci)
    for pos in (P.block + 5, P.L // 2 + 11, P.L - 40):
        print(f"[decode] unfilled cache case {ci} pos {pos}", flush=True)
        k2, v2 = k.clone(), v.clone()
        tail = k2[:, :, pos + 1:].shape
        k2[:, :, pos + 1:] = (3.0 * torch.randn(tail, generator=g) + 2.0).to(k.dtype)
        v2[:, :, pos + 1:] = (3.0 * torch.randn(tail, generator=g) - 1.0).to(v.dtype)
        dk2, dv2 = k2.cuda(), v2.cuda()
        st2 = pisa.block_stats(p, dq, dk2, dv2)
        qt = dq[:, :, pos].contiguous()
        idx = pisa.decode_topk(p, pos, qt, st)
        idx2 = pisa.decode_topk(p, pos, qt, st2)
        out, lse = pisa.decode_fwd(p, pos, qt, dk, dv, st, idx)
        out2, lse2 = pisa.decode_fwd(p, pos, qt, dk2, dv2, st2, idx2)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx2), f"pos {pos}: lists depend on slots after the token"
        assert torch.equal(out, out2) and torch.equal(lse, lse2), f"pos {pos}: output depends on later slots"
        qa, ka, va = (x.double().numpy() for x in (q, k2, v2))
        st_ref = po.block_stats(qa, ka, va, P)
        ref_idx = po.decode_select(qa[:, :, pos], st_ref, P, pos)
        assert np.array_equal(idx2.cpu().numpy().astype(np.int64), ref_idx)
        o_ref, l_ref = po.decode_attend(qa[:, :, pos], ka, va, st_ref, ref_idx, P, pos)
        _check(out2, lse2, o_ref, l_ref, tol, f"unfilled pos {pos}")


@pytest.mark.parametrize("w,d,dtype", [(256, 128, "bf16"), (100, 64, "bf16"), (64, 128, "f32")])
def test_decode_ring_buffer(w, d, dtype):
    kn = dict(B=1, Hq=4, Hkv=2, L=700, d=d, dtype=dtype, block=64, topk=0, window=w, taylor="none",
              causal=True)
    P = problem(kn)
    q, k, v = _inputs(kn, 3)
    p = pisa.make_params(**kn)
    kr = torch.zeros((1, 2, w, d), dtype=q.dtype)
    vr = torch.zeros_like(kr)
    tol = TOL[dtype]
    for pos in range(P.L):          # the ring as a decoder fills it
        kr[:, :, pos % w] = k[:, :, pos]
        vr[:, :, pos % w] = v[:, :, pos]
        if pos not in (0, w - 1, w, w + 17, P.L - 1):
            continue
        print(f"[decode] ring {w} pos {pos}", flush=True)
        out, lse = pisa.decode_fwd(p, pos, q[:, :, pos].contiguous().cuda(), kr.cuda(), vr.cuda(), ring=w)
        torch.cuda.synchronize()
        o_ref, l_ref = po.decode_ring(q[:, :, pos].double().numpy(), kr.double().numpy(),
                                      vr.double().numpy(), P, pos, w)
        _check(out, lse, o_ref, l_ref, tol, f"ring {w} pos {pos}")
