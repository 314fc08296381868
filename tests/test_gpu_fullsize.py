"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times.

The whole path runs on the GPU over the full problem. The CPU float64 oracle
recomputes what it can afford:
* for sampled (batch, query head) pairs, everything of that head: pooled
  selection vectors, block statistics and every selection row;
* the outputs of sampled tokens of that head: the first and last tokens, block
  boundaries, the ragged tail and seeded random tokens;
* the outputs of whole query blocks of that head, every row of them: the
  first block, the last (ragged where L is not a multiple of the block) and
  two seeded blocks in between (each row of them takes its Taylor terms in
  several batches of the kernel), with the mean-abs bar over those rows;
* for head (0, 0), every row of the head: outputs and lse of all L tokens,
  the oracle's attention split into chunks of 1024 tokens on a thread pool,
  max-abs per chunk and mean-abs over the whole head.
Bar: selections and pooled vectors bit-exact; outputs within max-abs 2e-2 /
mean-abs 2e-3 (bf16) or 1e-4 (fp32); lse within 1e-2 / 1e-5.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from gpu_common import TOL, problem
from oracle import pisa_oracle as po
from piecewise_attention_dit_amd import pisa
from piecewise_attention_dit_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _heads(wl):
    hs = [(0, 0), (wl.B - 1, wl.Hq - 1)]
    if wl.Hq > 2:
        hs.append((wl.B // 2, wl.Hq // 2 + 1))
    return sorted(set(hs))


def _blocks(wl, rng):
    n_blk = -(-wl.L // wl.block)
    mid = rng.choice(np.arange(1, n_blk - 1), size=2, replace=False)
    return sorted({0, n_blk - 1, *(int(x) for x in mid)})


def _tokens(wl, rng, n_random=12):
    L, bs = wl.L, wl.block
    t = {0, 1, L - 1, L - 2, bs - 1, bs, min(L - 1, 3 * bs + 5), ((L - 1) // bs) * bs}
    t |= set(int(x) for x in rng.integers(0, L, size=n_random))
    return np.array(sorted(x for x in t if 0 <= x < L), dtype=np.int64)


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_fullsize(name):
    wl = W.WORKLOADS[name]
    print(f"[fullsize] {name}: generating inputs", flush=True)
    q, k, v = W.make_inputs(wl)
    kn = wl.knobs()
    p = pisa.make_params(**kn)
    print(f"[fullsize] {name}: GPU path", flush=True)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    st = pisa.block_stats(p, dq, dk, dv)
    idx, cand = pisa.indexer_topk(p, dq, st)
    out, lse = pisa.sparse_attn_fwd(p, dq, dk, dv, st, idx)
    torch.cuda.synchronize()
    g_idx = idx.cpu().numpy()
    g_cand = cand.cpu().numpy() if cand is not None else None
    g_stats = {key: (t.cpu() if t is not None else None) for key, t in st.items()}
    del dq, dk, dv

    tol = TOL[wl.dtype]
    rng = np.random.default_rng(7)
    P1 = problem(dict(kn, B=1, Hq=1, Hkv=1))
    for (b, h) in _heads(wl):
        hk = h * wl.Hkv // wl.Hq
        qa = q[b:b + 1, h:h + 1].double().numpy()
        ka = k[b:b + 1, hk:hk + 1].double().numpy()
        va = v[b:b + 1, hk:hk + 1].double().numpy()
        print(f"[fullsize] {name}: oracle for b={b} h={h} (kv head {hk})", flush=True)
        ref = po.block_stats(qa, ka, va, P1)
        # pooled selection vectors and statistics of this head
        np.testing.assert_array_equal(g_stats["qsel"][b, h].double().numpy(), ref["qsel"][0, 0])
        np.testing.assert_array_equal(g_stats["ksel"][b, hk].double().numpy(), ref["ksel"][0, 0])
        if wl.taylor != "none":
            np.testing.assert_array_equal(g_stats["kbar"][b, hk].double().numpy(),
                                          po.rne(ref["kbar"][0, 0], "f32"))
            vs = ref["vsum"][0, 0]
            err = np.abs(g_stats["vsum"][b, hk].double().numpy() - vs).max() / np.abs(vs).max()
            assert err < 1e-5, f"vsum relative error {err}"
        if wl.taylor == "order1":
            H = ref["H"][0, 0]                                              # [n_blk, c, e]
            HT = g_stats["HT"][b, hk].double().numpy()                      # [n_blk, e, c]
            num = np.linalg.norm((np.swapaxes(HT, -1, -2) - H).reshape(len(H), -1), axis=1)
            den = np.linalg.norm(H.reshape(len(H), -1), axis=1) + 1e-30
            assert (num / den).max() < tol["H"], f"H relative error {(num / den).max()}"
        # every selection row of this head
        r_idx, r_cand = po.select(qa, ref, P1)
        gi = g_idx[b, h].astype(np.int64)
        bad = np.argwhere((gi != r_idx[0, 0]).any(axis=-1)).ravel()
        assert len(bad) == 0, f"{len(bad)} rows differ, first {bad[:5].tolist()}: " \
                              f"gpu {gi[bad[0]].tolist()} oracle {r_idx[0, 0, bad[0]].tolist()}"
        if g_cand is not None:
            assert np.array_equal(g_cand[b, h].astype(np.int64), r_cand[0, 0]), "proxy lists differ"
        # outputs of sampled tokens
        toks = _tokens(wl, rng)
        o_ref, l_ref = po.attend_tokens(qa, ka, va, ref, r_idx, P1, 0, 0, toks)
        o_gpu = out[b, h, toks].cpu().double().numpy()
        l_gpu = lse[b, h, toks].cpu().double().numpy()
        assert np.isfinite(o_gpu).all()
        d = np.abs(o_gpu - o_ref)
        print(f"[fullsize] {name} b={b} h={h}: {len(toks)} tokens max_abs={d.max():.3e} "
              f"mean_abs={d.mean():.3e}", flush=True)
        assert d.max() <= tol["max_abs"], f"max abs error {d.max()}"
        assert d.mean() <= tol["mean_abs"], f"mean abs error {d.mean()}"
        assert np.abs(l_gpu - l_ref).max() <= tol["lse"], f"lse error {np.abs(l_gpu - l_ref).max()}"
        if (b, h) == (0, 0):   # the whole head, every row
            chunks = [np.arange(t0, min(wl.L, t0 + 1024)) for t0 in range(0, wl.L, 1024)]
            print(f"[fullsize] {name}: oracle attention of the whole head ({wl.L} rows, "
                  f"{len(chunks)} chunks)", flush=True)
            with ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
                refs = list(ex.map(lambda tk: po.attend_tokens(qa, ka, va, ref, r_idx, P1, 0, 0, tk), chunks))
            o_all = out[b, h].cpu().double().numpy()
            l_all = lse[b, h].cpu().double().numpy()
            assert np.isfinite(o_all).all()
            s_abs, n_el = 0.0, 0
            for tk, (o_ref, l_ref) in zip(chunks, refs):
                d = np.abs(o_all[tk] - o_ref)
                assert d.max() <= tol["max_abs"], f"rows {tk[0]}..{tk[-1]}: max abs error {d.max()}"
                assert np.abs(l_all[tk] - l_ref).max() <= tol["lse"], f"rows {tk[0]}..{tk[-1]}: lse error"
                s_abs += d.sum()
                n_el += d.size
            print(f"[fullsize] {name} b=0 h=0 whole head: mean_abs={s_abs / n_el:.3e}", flush=True)
            assert s_abs / n_el <= tol["mean_abs"], f"whole head: mean abs error {s_abs / n_el}"
        # whole query blocks, every row
        for i in _blocks(wl, rng):
            toks = np.arange(i * wl.block, min(wl.L, (i + 1) * wl.block))
            o_ref, l_ref = po.attend_tokens(qa, ka, va, ref, r_idx, P1, 0, 0, toks)
            o_gpu = out[b, h, toks].cpu().double().numpy()
            l_gpu = lse[b, h, toks].cpu().double().numpy()
            assert np.isfinite(o_gpu).all()
            d = np.abs(o_gpu - o_ref)
            print(f"[fullsize] {name} b={b} h={h} query block {i} ({len(toks)} rows): "
                  f"max_abs={d.max():.3e} mean_abs={d.mean():.3e}", flush=True)
            assert d.max() <= tol["max_abs"], f"block {i}: max abs error {d.max()}"
            assert d.mean() <= tol["mean_abs"], f"block {i}: mean abs error {d.mean()}"
            assert np.abs(l_gpu - l_ref).max() <= tol["lse"], f"block {i}: lse error"
