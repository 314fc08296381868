"""pisa_decode_fwd_noalloc (split-K partials in the library's fixed scratch,
for callers that cannot allocate) against pisa_decode_fwd (caller
workspace): the two run the same kernels, so outputs and lse must agree bit
for bit.  Two calls in a row on one device, the second on a smaller problem,
so the second runs over the first call's leftover partials."""
import numpy as np
import pytest
import torch

from piecewise_attention_dit_amd import pisa
from piecewise_attention_dit_amd import workloads as W

pytestmark = pytest.mark.gpu

CALLS = [
    dict(B=4, Hq=32, Hkv=8, L=2048, d=128, dtype="bf16", block=64, topk=4, window=256, taylor="order1"),
    dict(B=1, Hq=4, Hkv=2, L=700, d=64, dtype="bf16", block=64, topk=2, window=100, taylor="order0"),
]


def _case(kn, seed):
    kn = dict(kn, causal=True)
    wl = W.Workload("noalloc", recipe="gauss", **kn)
    q, k, v = W.make_inputs(wl, seed=seed)
    p = pisa.make_params(**kn)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    st = pisa.block_stats(p, dq, dk, dv)
    pos = kn["L"] - 5
    qt = dq[:, :, pos].contiguous()
    idx = pisa.decode_topk(p, pos, qt, st)
    return p, pos, qt, dk, dv, st, idx


def test_noalloc_matches_workspace_entry():
    assert pisa.workspace_size(pisa.make_params(**dict(CALLS[0], causal=True)), 3) > \
        pisa.workspace_size(pisa.make_params(**dict(CALLS[1], causal=True)), 3)
    for ci, kn in enumerate(CALLS):
        print(f"[noalloc] call {ci}: {kn}", flush=True)
        p, pos, qt, dk, dv, st, idx = _case(kn, 21 + ci)
        ref_o, ref_l = pisa.decode_fwd(p, pos, qt, dk, dv, st, idx)
        out, lse = pisa.decode_fwd_noalloc(p, pos, qt, dk, dv, st, idx)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        assert torch.equal(out, ref_o), f"call {ci}: outputs differ"
        assert torch.equal(lse, ref_l), f"call {ci}: lse differs"
    # a ring-buffer step through the fixed scratch as well
    kn = dict(B=1, Hq=4, Hkv=2, L=300, d=128, dtype="bf16", block=64, topk=0, window=64, taylor="none",
              causal=True)
    p = pisa.make_params(**kn)
    g = torch.Generator().manual_seed(5)
    q = torch.randn(1, 4, 128, generator=g).to(torch.bfloat16).cuda()
    kr = torch.randn(1, 2, 64, 128, generator=g).to(torch.bfloat16).cuda()
    vr = torch.randn(1, 2, 64, 128, generator=g).to(torch.bfloat16).cuda()
    ref_o, ref_l = pisa.decode_fwd(p, 200, q, kr, vr, ring=64)
    out, lse = pisa.decode_fwd_noalloc(p, 200, q, kr, vr, ring=64)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
