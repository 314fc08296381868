"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded inputs, and compare them."""
from __future__ import annotations

import numpy as np
import torch

from oracle import pisa_oracle as po
from piecewise_attention_dit_amd import pisa

# tolerances (float outputs), bit-exact for selections and pooled vectors
TOL = {"bf16": dict(max_abs=2e-2, mean_abs=2e-3, lse=1e-2, H=1e-2),
       "f32": dict(max_abs=1e-4, mean_abs=1e-4, lse=1e-5, H=1e-5)}


def problem(knobs: dict) -> po.Problem:
    return po.Problem.from_knobs(**knobs)


def run_gpu(knobs: dict, q, k, v, diag: bool = True) -> dict:
    """The three library calls on cuda:0; returns CPU copies of everything."""
    p = pisa.make_params(**knobs)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    st = pisa.block_stats(p, dq, dk, dv)
    dg = torch.zeros(16, dtype=torch.int32, device="cuda") if diag else None
    idx, cand = pisa.indexer_topk(p, dq, st, diag=dg)
    out, lse = pisa.sparse_attn_fwd(p, dq, dk, dv, st, idx)
    torch.cuda.synchronize()
    res = dict(stats={k2: (t.cpu() if t is not None else None) for k2, t in st.items()},
               idx=idx.cpu(), cand=cand.cpu() if cand is not None else None, O=out.cpu(), lse=lse.cpu(),
               diag=dg.cpu() if dg is not None else None)
    return res


def to64(t):
    return t.double().numpy()


def compare_stats(g: dict, st: dict, P: po.Problem):
    gs = g["stats"]
    np.testing.assert_array_equal(to64(gs["qsel"]), st["qsel"], err_msg="qsel not bit-exact")
    np.testing.assert_array_equal(to64(gs["ksel"]), st["ksel"], err_msg="ksel not bit-exact")
    if P.taylor != "none":
        np.testing.assert_array_equal(to64(gs["kbar"]), po.rne(st["kbar"], "f32"),
                                      err_msg="kbar is not the fp32 rounding of the mean")
        vs = st["vsum"]
        err = np.abs(to64(gs["vsum"]) - vs).max() / max(1e-30, np.abs(vs).max())
        assert err < 1e-5, f"vsum relative error {err}"
    if P.taylor == "order1":
        H = st["H"]                                    # [.., c, e]
        HT = to64(gs["HT"])                            # [.., e, c]
        num = np.linalg.norm((np.swapaxes(HT, -1, -2) - H).reshape(-1, P.d * P.d), axis=1)
        den = np.linalg.norm(H.reshape(-1, P.d * P.d), axis=1) + 1e-30
        rel = (num / den).max()
        assert rel < TOL[P.dtype]["H"], f"H relative Frobenius error {rel}"
    if P.taylor == "hybrid":
        # non-causal: one mean [B, Hkv, c, e]; causal: one per lo [B, Hkv, n_blk, c, e]
        Hb = st["Hpre"] if P.causal else st["Hbar"]
        HbT = to64(gs["HT"])
        num = np.linalg.norm((np.swapaxes(HbT, -1, -2) - Hb).reshape(-1, P.d * P.d), axis=1)
        den = np.linalg.norm(Hb.reshape(-1, P.d * P.d), axis=1) + 1e-30
        # the empty prefix (lo = 0) is exactly zero on both sides
        rel = (num / den)[den > 1e-20].max()
        assert rel < TOL[P.dtype]["H"], f"Hbar relative Frobenius error {rel}"
        if P.causal:
            assert not HbT[:, :, 0].any(), "Hbar(lo = 0) must be zero"
    if P.route_lambda > 0:
        err = np.abs(to64(gs["mcov"]) - st["M"])
        tol = MCOV_REL * st["M"].max(axis=-1, keepdims=True) + 1e-30
        assert (err <= tol).all(), f"covariance norm error {(err / tol).max()} x tolerance"


# covariance norms: the HIP path forms H_j from exact products in fp32 (and
# Hbar in fp32), the oracle in float64; relative to the largest norm of the head
MCOV_REL = 1e-4


def compare_idx_routed(g: dict, ref: dict, P: po.Problem, q: np.ndarray) -> np.ndarray:
    """Selections under covariance-aware routing.  The HIP path selects
    exactly for its own covariance norms, which agree with the oracle's to
    MCOV_REL: where a row's top set is decided by more than that, the two
    selections must be identical; otherwise the HIP path's set must be a
    valid top set for the oracle's scores up to that margin.  Returns a mask
    [B, Hq, n_rows] of rows that are identical."""
    st = ref["stats"]
    gi = g["idx"].numpy().astype(np.int64)
    oi = ref["idx"]
    same = (gi == oi).all(axis=-1)
    lam = float(np.float32(P.route_lambda))
    gc = g["cand"].numpy().astype(np.int64) if g["cand"] is not None else None
    for (b, h, r) in np.argwhere(~same):
        hk = h * P.Hkv // P.Hq
        slack = 2.0 * lam * MCOV_REL * st["M"][b, hk].max() + 1e-9
        if P.pivot:
            gm = r // P.group
            if gc is not None and not np.array_equal(gc[b, h, gm], ref["cand"][b, h, gm]):
                continue            # the proxy stage differs: checked below
            cands = ref["cand"][b, h, gm]
            cands = cands[cands >= 0]
            vec = q[b, h, r]
        else:
            nc = po.row_geometry(P, r)[2]
            cands = np.arange(po.sink_count(P, nc), nc)
            vec = st["qsel"][b, h, r]
        score = st["ksel"][b, hk][cands] @ vec + lam * st["M"][b, hk][cands]
        kept = set(int(j) for j in gi[b, h, r] if j >= 0)
        ins = np.array([score[i] for i, j in enumerate(cands) if j in kept])
        outs = np.array([score[i] for i, j in enumerate(cands) if j not in kept])
        if len(ins) and len(outs):
            assert ins.min() >= outs.max() - slack, f"row {(b, h, r)} is not a top set within the margin"
    if gc is not None:
        for (b, h, gm) in np.argwhere(~(gc == ref["cand"]).all(axis=-1)):
            hk = h * P.Hkv // P.Hq
            slack = 2.0 * lam * MCOV_REL * st["M"][b, hk].max() + 1e-9
            nc = po.group_candidates(P, gm)
            cands = np.arange(po.sink_count(P, nc), nc)
            score = st["ksel"][b, hk][cands] @ st["qsel"][b, h, gm] + lam * st["M"][b, hk][cands]
            kept = set(int(j) for j in gc[b, h, gm] if j >= 0)
            ins = np.array([score[i] for i, j in enumerate(cands) if j in kept])
            outs = np.array([score[i] for i, j in enumerate(cands) if j not in kept])
            if len(ins) and len(outs):
                assert ins.min() >= outs.max() - slack, f"proxy {(b, h, gm)} is not a top set within the margin"
    frac = 1.0 - same.mean()
    assert frac <= 0.01, f"{frac:.3%} of the rows differ"
    return same


def compare_idx(g: dict, idx: np.ndarray, cand, rows=None):
    gi = g["idx"].numpy().astype(np.int64)
    if rows is None:
        bad = np.argwhere((gi != idx).any(axis=-1))
        assert len(bad) == 0, f"{len(bad)} rows differ, first {bad[:5].tolist()}: " \
                              f"gpu {gi[tuple(bad[0])]} oracle {idx[tuple(bad[0])]}"
    else:
        for (b, h, r) in rows:
            assert np.array_equal(gi[b, h, r], idx[b, h, r]), (b, h, r, gi[b, h, r], idx[b, h, r])
    if cand is not None:
        gc = g["cand"].numpy().astype(np.int64)
        assert np.array_equal(gc, cand), "PIVOT proxy lists differ"


def compare_out(g: dict, O: np.ndarray, lse: np.ndarray, P: po.Problem, sel=None):
    go, gl = to64(g["O"]), g["lse"].double().numpy()
    if sel is not None:
        go, gl, O, lse = go[sel], gl[sel], O[sel], lse[sel]
    t = TOL[P.dtype]
    d = np.abs(go - O)
    assert np.isfinite(go).all(), "non-finite output"
    assert d.max() <= t["max_abs"], f"max abs error {d.max()}"
    assert d.mean() <= t["mean_abs"], f"mean abs error {d.mean()}"
    dl = np.abs(gl - lse).max()
    assert dl <= t["lse"], f"lse error {dl}"
    return d.max(), d.mean()
