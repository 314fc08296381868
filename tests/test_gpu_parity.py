"""GPU parity: the HIP path (through the C ABI) against the CPU float64 oracle.

Bar: pooled selection vectors and block selections bit-exact; outputs within
max-abs 2e-2 / mean-abs 2e-3 (bf16) or 1e-4 (fp32); lse within 1e-2 / 1e-5.
"""
import numpy as np
import pytest
import torch

from gpu_common import compare_idx, compare_idx_routed, compare_out, compare_stats, problem, run_gpu
from oracle import pisa_oracle as po
from piecewise_attention_dit_amd import workloads as W

pytestmark = pytest.mark.gpu


def _check_case(knobs, q, k, v):
    P = problem(knobs)
    qa, ka, va = (x.double().numpy() for x in (q, k, v))
    print(f"[parity] {knobs}", flush=True)
    g = run_gpu(knobs, q, k, v)
    ref = po.run(qa, ka, va, P)
    compare_stats(g, ref["stats"], P)
    O_ref, lse_ref = ref["O"], ref["lse"]
    if P.route_lambda > 0:
        same = compare_idx_routed(g, ref, P, qa)
        # a row whose selection differs (decided within the covariance norms'
        # margin) is checked against the oracle attending with the GPU's own list
        gidx = g["idx"].numpy().astype(np.int64)
        O_ref, lse_ref = O_ref.copy(), lse_ref.copy()
        for (b, h, r) in np.argwhere(~same):
            toks = [int(r)] if P.pivot else list(range(r * P.block, min(P.L, (r + 1) * P.block)))
            O_ref[b, h, toks], lse_ref[b, h, toks] = po.attend_tokens(qa, ka, va, ref["stats"], gidx, P,
                                                                      int(b), int(h), toks)
        print(f"[parity] routing: {int((~same).sum())} of {same.size} rows differ within the margin "
              f"(outputs checked with their own lists)", flush=True)
    else:
        compare_idx(g, ref["idx"], ref["cand"])
    mx, mn = compare_out(g, O_ref, lse_ref, P)
    print(f"[parity] ok max_abs={mx:.3e} mean_abs={mn:.3e} diag={g['diag'][:3].tolist()}", flush=True)
    return g, ref


@pytest.mark.parametrize("name", sorted(W.PARITY_CASES))
def test_parity_cases(name):
    wl = W.PARITY_CASES[name]
    q, k, v = W.make_inputs(wl)
    _check_case(wl.knobs(), q, k, v)


@pytest.mark.parametrize("kw", [
    dict(L=1, block=64, topk=1),                                  # one token
    dict(L=50, block=64, topk=1, causal=True, window=8),          # less than a block
    dict(L=700, block=64, topk=0, taylor="order1"),               # all blocks Taylor
    dict(L=700, block=64, topk=11, taylor="order1"),              # k >= n_blk: dense
    dict(L=700, block=128, topk=2, Hq=8, Hkv=1, causal=True),     # GQA 8
    dict(L=700, block=64, topk=3, Hq=4, Hkv=2, causal=True, window=200),   # GQA 2 + window
    dict(L=900, block=64, topk=4, group=1, n_cand=64, causal=True, taylor="none"),  # dense per-token
    dict(L=900, block=64, topk=3, group=4, n_cand=6, causal=True, window=150, taylor="order1"),
    dict(L=640, block=128, topk=2, group=8, n_cand=5, causal=False, taylor="order0"),
    dict(L=600, block=64, topk=2, d=64, Hq=2, Hkv=2, taylor="order1", dtype="f32", causal=True,
         window=100),
    dict(L=700, block=64, topk=0, taylor="hybrid"),               # hybrid, all blocks Taylor
    dict(L=777, block=128, topk=1, d=64, taylor="hybrid"),        # hybrid, d 64 with 128-blocks
    dict(L=300, block=128, topk=1, d=128, taylor="hybrid", dtype="f32"),
    dict(L=700, block=64, topk=0, sink=2, causal=True, window=130, taylor="order0"),  # sinks only
    dict(L=600, block=64, topk=2, d=64, dtype="f32", causal=True, window=100, sink=2),
    dict(L=500, block=64, topk=2, d=64, group=4, n_cand=5, dtype="f32", causal=True, sink=3,
         taylor="none"),
    dict(L=900, block=64, topk=3, group=4, n_cand=6, causal=True, window=150, sink=20,
         taylor="order1"),                                        # sinks beyond most rows' reach
    dict(L=600, block=64, topk=2, d=64, dtype="f32", route_lambda=0.005),   # routing, fp32
    dict(L=500, block=64, topk=2, d=64, group=4, n_cand=5, dtype="f32", causal=False,
         taylor="order0", route_lambda=0.01),                    # routing, fp32 PIVOT
    dict(L=777, block=128, topk=1, d=64, taylor="order1", route_lambda=0.02),
    # causal hybrid order (the mean over each row's candidates): fp32 block rows
    # and PIVOT rows, bf16 d 64 with several block rows per workgroup
    dict(L=600, block=64, topk=2, d=64, dtype="f32", causal=True, window=100, taylor="hybrid"),
    dict(L=500, block=64, topk=2, d=64, group=4, n_cand=5, dtype="f32", causal=True, taylor="hybrid"),
    dict(L=1300, block=64, topk=2, d=64, causal=True, window=130, taylor="hybrid"),
    dict(L=1500, block=128, topk=1, d=128, causal=True, taylor="hybrid"),
    # PIVOT rows without a Taylor tail (key-gathered kernel): GQA 8 with a
    # window, one head per kv head with d 64 and 128-token blocks, non-causal
    # GQA 2, and rows whose lists repeat the whole proxy list
    dict(L=900, block=64, topk=3, group=4, n_cand=6, causal=True, window=150, taylor="none", Hq=8, Hkv=1),
    dict(L=1300, block=128, topk=2, group=8, n_cand=5, causal=True, taylor="none", d=64, Hq=2, Hkv=2),
    dict(L=700, block=64, topk=3, group=2, n_cand=6, causal=False, taylor="none", Hq=4, Hkv=2),
    dict(L=1100, block=64, topk=5, group=8, n_cand=5, causal=True, window=64, taylor="none", Hq=4, Hkv=2, sink=1),
    # pools of 32 tokens at d 64 (GQA 8), of 256 tokens (one query head per
    # kv head, 128-token blocks, a window), and a sequence shorter than one pool
    dict(L=700, block=64, topk=3, group=4, n_cand=6, causal=True, taylor="none", d=64, Hq=8, Hkv=1),
    dict(L=1500, block=128, topk=2, group=8, n_cand=4, causal=True, window=300, taylor="none", Hq=2, Hkv=2),
    dict(L=100, block=64, topk=1, group=4, n_cand=2, causal=True, taylor="none", Hq=4, Hkv=1),
    # kept lists longer than 64 blocks (entries past 64 read from LDS), and
    # every block kept (the dense case through the sparse kernel)
    dict(L=64 * 90 - 17, block=64, topk=75, d=64, taylor="order1"),
    dict(L=128 * 70, block=128, topk=70, d=128, taylor="order1", causal=True, window=300),
    dict(L=128 * 80, block=128, topk=80, d=128, taylor="order1"),
    # d 64 first order takes four Taylor entries per barrier: two batches of
    # entries, the last group short
    dict(L=1500, block=64, topk=2, d=64, taylor="order1"),
    dict(L=1700, block=64, topk=2, d=64, taylor="order1", causal=True, window=200),
    dict(L=2900, block=128, topk=2, d=64, taylor="order1"),
    # fp32 block rows at d 128 (8 x 8 moment tiles per thread, two output
    # features per lane), causal GQA with a window, and more than 64 Taylor
    # blocks (two Taylor batches of the row-block kernel)
    dict(L=700, block=128, topk=2, d=128, dtype="f32"),
    dict(L=650, block=64, topk=3, d=128, dtype="f32", causal=True, window=100, Hq=4, Hkv=2),
    dict(L=64 * 80 - 9, block=64, topk=2, d=64, dtype="f32"),
])
def test_edge_cases(kw):
    base = dict(B=1, Hq=2, Hkv=2, L=256, d=128, dtype="bf16", block=64, topk=2, window=0, group=0,
                n_cand=0, causal=False, taylor="order1")
    base.update(kw)
    wl = W.Workload("edge", **{k2: v2 for k2, v2 in base.items() if k2 != "name"}, recipe="gauss")
    q, k, v = W.make_inputs(wl, seed=5)
    _check_case(base, q, k, v)


def _planted(d=128, bs=64, nblk=8, dtype=torch.bfloat16):
    """Query block 0 is constant with pooled vector p = (1, 2^-30, 1, -1, 0...);
    key blocks 1, 2, 3 are constant with (1,0..), (1, 2^-30, 0..), (.5, 0, .5, 0..):
    exact scores 1, 1 + 2^-60, 1 (the first and last tie exactly, the middle one
    exceeds them by less than float64 resolves); blocks 5 and 6 are bitwise
    copies of block 1; every other key block scores -1."""
    L = bs * nblk
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 1, L, d, generator=g)
    k = torch.zeros(1, 1, L, d)
    k[0, 0, :, 0] = -1.0
    pvec = torch.zeros(d)
    pvec[0], pvec[1], pvec[2], pvec[3] = 1.0, 2.0 ** -30, 1.0, -1.0
    q[0, 0, :bs] = pvec
    blk = lambda j: slice(j * bs, (j + 1) * bs)
    k[0, 0, blk(1)] = 0.0
    k[0, 0, blk(1), 0] = 1.0
    k[0, 0, blk(2)] = 0.0
    k[0, 0, blk(2), 0], k[0, 0, blk(2), 1] = 1.0, 2.0 ** -30
    k[0, 0, blk(3)] = 0.0
    k[0, 0, blk(3), 0], k[0, 0, blk(3), 2] = 0.5, 0.5
    k[0, 0, blk(5)] = k[0, 0, blk(1)]
    k[0, 0, blk(6)] = k[0, 0, blk(1)]
    v = torch.randn(1, 1, L, d, generator=g)
    return q.to(dtype), k.to(dtype), v.to(dtype)


@pytest.mark.parametrize("topk,want", [(1, [2]), (2, [1, 2]), (3, [1, 2, 3]), (4, [1, 2, 3, 5])])
def test_exact_tie_paths(topk, want):
    q, k, v = _planted()
    knobs = dict(B=1, Hq=1, Hkv=1, L=q.shape[2], d=128, dtype="bf16", block=64, topk=topk, window=0,
                 group=0, n_cand=0, causal=False, taylor="order1")
    g, ref = _check_case(knobs, q, k, v)
    assert g["idx"][0, 0, 0].tolist() == want
    assert ref["idx"][0, 0, 0].tolist() == want
    assert int(g["diag"][1]) >= 1          # the exact re-scoring path ran


def test_deterministic_bitwise():
    wl = W.PARITY_CASES["llm_swa_s"]
    q, k, v = W.make_inputs(wl)
    a = run_gpu(wl.knobs(), q, k, v)
    b = run_gpu(wl.knobs(), q, k, v)
    for key in ("idx", "O", "lse"):
        assert torch.equal(a[key], b[key]), key
    for key, t in a["stats"].items():
        if t is not None:
            assert torch.equal(t, b["stats"][key]), key


def _wide_spread(d, bs, L, dtype=torch.bfloat16):
    """Q and K with one feature column per block that a plain float64 sum gets
    wrong: tokens 0, 16 and 32 of the block hold 2^60, 1 and -2^60 (its other
    tokens 0), so the correctly rounded sum is 1 and the mean 1 / block, while
    summing them in that order in float64 loses the 1 and gives 0.  One lane
    sums those tokens in the key kernel (and, for d = 128, in the query
    kernel), so its exponent-spread certificate fails (60 bits) and the exact
    fallback decides the result."""
    g = torch.Generator().manual_seed(11)
    q = torch.randn(1, 2, L, d, generator=g)
    k = torch.randn(1, 2, L, d, generator=g)
    v = torch.randn(1, 2, L, d, generator=g)
    for x in (q, k):
        for j in range(L // bs):
            f = 5 + j % 3
            x[:, :, j * bs:(j + 1) * bs, f] = 0.0
            x[:, :, j * bs + 0, f] = 2.0 ** 60
            x[:, :, j * bs + 16, f] = 1.0
            x[:, :, j * bs + 32, f] = -(2.0 ** 60)
    return q.to(dtype), k.to(dtype), v.to(dtype)


@pytest.mark.parametrize("d,bs", [(128, 64), (128, 128), (64, 64), (64, 128)])
def test_pooling_exact_beyond_float64(d, bs):
    from piecewise_attention_dit_amd import pisa
    L = 4 * bs
    q, k, v = _wide_spread(d, bs, L)
    knobs = dict(B=1, Hq=2, Hkv=2, L=L, d=d, dtype="bf16", block=bs, topk=1, window=0, group=0,
                 n_cand=0, causal=False, taylor="order1")
    P = problem(knobs)
    print(f"[parity] wide exponent spread d={d} block={bs}", flush=True)
    ref = po.block_stats(*(x.double().numpy() for x in (q, k, v)), P)
    # the case is sensitive: the pooled value is 1 / block, not the 0 of a plain sum
    assert ref["ksel"][0, 0, 0, 5] == 1.0 / bs and ref["qsel"][0, 0, 0, 5] == 1.0 / bs
    p = pisa.make_params(**knobs)
    st = pisa.block_stats(p, q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    g = dict(stats={key: (t.cpu() if t is not None else None) for key, t in st.items()})
    compare_stats(g, ref, P)


def _messy_lists(idx, P, rng, width):
    """Kept lists as a caller might pass them (reused from another layer):
    the valid entries of idx plus a repeat, negative values, blocks past the
    sequence, beyond the kernels' 1024-block range, and (causal) blocks of the
    row's window range.  Block rows in shuffled order; PIVOT rows keep their
    valid entries ascending (a precondition there) with the rest interleaved.
    Returns (messy, filtered): filtered is what the guard must keep."""
    B, Hq, R, _ = idx.shape
    messy = np.full((B, Hq, R, width), -1, dtype=np.int64)
    filt = np.full((B, Hq, R, width), -1, dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            for r in range(R):
                own, lo, nc = po.row_geometry(P, r)
                valid = [int(j) for j in idx[b, h, r] if j >= 0]
                wild = [-5, 1024 + r % 7, 5000, P.n_blk, nc, -2 ** 31, P.n_blk + 40]
                if P.causal:
                    wild += [own, lo]
                extra = valid[:1] + [int(x) for x in rng.permutation(wild)]
                extra = extra[:width - len(valid)]
                if P.pivot:
                    ent = list(valid)
                    for x in extra:
                        ent.insert(int(rng.integers(0, len(ent) + 1)), x)
                else:
                    ent = [int(x) for x in rng.permutation(valid + extra)]
                messy[b, h, r, :len(ent)] = ent
                filt[b, h, r, :len(valid)] = sorted(set(valid))
    return messy, filt


@pytest.mark.parametrize("name", ["llm_swa_s", "video_dit_s", "llm_pivot_s", "llm_pivot_s_hyb",
                                  "llm_swa_s_hyb_w", "tiny_f32_ragged"])
def test_reused_lists_are_filtered(name):
    """HyLRA page, section 2.3: a tolerant layer attends with another layer's
    lists.  The attention call keeps only the entries that are candidates of
    each row and must equal the oracle on the filtered lists."""
    from piecewise_attention_dit_amd import pisa
    wl = W.PARITY_CASES[name]
    q, k, v = W.make_inputs(wl, seed=9)
    kn = wl.knobs()
    P = problem(kn)
    qa, ka, va = (x.double().numpy() for x in (q, k, v))
    st_ref = po.block_stats(qa, ka, va, P)
    idx, _ = po.select(qa, st_ref, P)
    width = P.klist + 7
    messy, filt = _messy_lists(idx, P, np.random.default_rng(31), width)
    # the attention call reads lists of that width (n_cand only bounds the
    # PIVOT indexer's lists, which this call does not use)
    kw = dict(kn, topk=width, sink=0, n_cand=max(kn["n_cand"], width) if kn["group"] else kn["n_cand"])
    Pw = problem(kw)
    print(f"[parity] reused lists with wild entries: {name} width {width}", flush=True)
    p = pisa.make_params(**kn)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    st = pisa.block_stats(p, dq, dk, dv)
    pw = pisa.make_params(**kw)
    out, lse = pisa.sparse_attn_fwd(pw, dq, dk, dv, st, torch.from_numpy(messy.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    O_ref, lse_ref = po.attention(qa, ka, va, st_ref, filt, Pw)
    mx, mn = compare_out(dict(O=out.cpu(), lse=lse.cpu()), O_ref, lse_ref, Pw)
    print(f"[parity] ok max_abs={mx:.3e} mean_abs={mn:.3e}", flush=True)
