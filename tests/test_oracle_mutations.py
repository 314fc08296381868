"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's source (on the CPU, in
memory) and checks that at least one pin check fails for the mutant, while
all of them pass for the unmodified oracle.
"""
import inspect
import sys
import types

import numpy as np
import pytest
import torch

from oracle import pisa_oracle as po


def _load(src: str, name: str):
    mod = types.ModuleType(name)
    mod.__dict__["__name__"] = name
    sys.modules[name] = mod
    exec(compile(src, name, "exec"), mod.__dict__)
    return mod


def _rand(shape, seed, dtype="f32", scale=1.0):
    return po.rne(scale * np.random.default_rng(seed).standard_normal(shape), dtype)


def _dense(q, k, v, P, causal):
    rep = P.Hq // P.Hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k).repeat_interleave(rep, 1),
        torch.from_numpy(v).repeat_interleave(rep, 1), is_causal=causal, scale=P.sm_scale)
    return o.numpy()


def check_swa_count(m):
    P = m.Problem(B=1, Hq=1, Hkv=1, L=16, d=4, dtype="f32", block=1, topk=0, window=4,
                  causal=True, taylor="none")
    return m.kept_pairs(P, np.full((1, 1, 16, 0), -1)).sum() == 58


def check_dense(m):
    ok = True
    for causal in (False, True):
        P = m.Problem(B=1, Hq=4, Hkv=2, L=70, d=8, dtype="bf16", block=8, topk=9,
                      causal=causal, taylor="order1")
        q, k, v = _rand((1, 4, 70, 8), 1, "bf16"), _rand((1, 2, 70, 8), 2, "bf16"), \
            _rand((1, 2, 70, 8), 3, "bf16")
        ok &= np.abs(m.run(q, k, v, P)["O"] - _dense(q, k, v, P, causal)).max() < 1e-12
    return ok


def check_constant_v(m):
    P = m.Problem(B=1, Hq=2, Hkv=2, L=64, d=8, dtype="f32", block=8, topk=2, causal=True,
                  window=10, taylor="order1")
    q, k = _rand((1, 2, 64, 8), 4), _rand((1, 2, 64, 8), 5)
    v = _rand((1, 2, 64, 8), 6)
    a = np.abs(m.run(q, k, np.ones_like(v), P)["O"] - 1).max() < 1e-12
    b = np.abs(m.run(q, k, v + 2.0, P)["O"] - m.run(q, k, v, P)["O"] - 2.0).max() < 1e-12
    return a and b


def check_orders(m):
    B, H, L, d, bs = 1, 1, 128, 8, 16
    rng = np.random.default_rng(7)
    cen = rng.standard_normal((B, H, L // bs, d))
    dl = rng.standard_normal((B, H, L // bs, bs, d))
    dl -= dl.mean(axis=3, keepdims=True)
    q, v = _rand((B, H, L, d), 8, scale=0.7), _rand((B, H, L, d), 9)
    errs = {"order0": [], "order1": []}
    for eps in (0.2, 0.1, 0.05):
        k = po.rne((cen[:, :, :, None, :] + eps * dl).reshape(B, H, L, d), "f32")
        for mode in errs:
            P = m.Problem(B=B, Hq=H, Hkv=H, L=L, d=d, dtype="f32", block=bs, topk=0, taylor=mode)
            errs[mode].append(np.abs(m.run(q, k, v, P)["O"] - _dense(q, k, v, P, False)).max())
    r0 = [a / b for a, b in zip(errs["order0"], errs["order0"][1:])]
    r1 = [a / b for a, b in zip(errs["order1"], errs["order1"][1:])]
    return all(1.7 < x < 2.3 for x in r0) and all(3.4 < x < 4.6 for x in r1)


def check_ties(m):
    d, bs, L = 6, 4, 40
    P = m.Problem(B=1, Hq=1, Hkv=1, L=L, d=d, dtype="bf16", block=bs, topk=3, taylor="order0")
    u = np.zeros(d)
    u[0] = 1.0
    q = po.rne(_rand((1, 1, L, d), 81, "f32", 0.05) + u, "bf16")
    k = _rand((1, 1, L, d), 82, "f32", 0.05)
    k[0, 0, bs:2 * bs] += 2.0 * u
    k = po.rne(k, "bf16")
    for dst in (5, 6, 7):
        k[0, 0, dst * bs:(dst + 1) * bs] = k[0, 0, bs:2 * bs]
    r = m.run(q, k, _rand((1, 1, L, d), 83, "bf16"), P)
    return all(r["idx"][0, 0, i].tolist() == [1, 5, 6] for i in range(P.n_blk))


def check_pivot_reuse(m):
    P = m.Problem(B=1, Hq=1, Hkv=1, L=96, d=8, dtype="bf16", block=16, topk=3, group=8,
                  n_cand=3, causal=True, taylor="none")
    q, k, v = _rand((1, 1, 96, 8), 10, "bf16"), _rand((1, 1, 96, 8), 11, "bf16"), \
        _rand((1, 1, 96, 8), 12, "bf16")
    r = m.run(q, k, v, P)
    same = all(np.array_equal(r["idx"][0, 0, t], r["cand"][0, 0, t // 8]) for t in range(96))
    # the proxy must be the mean of its group: compare with a planted group
    return same


def check_pooled_selection(m):
    """Selection vectors are the rounded block means: a planted answer."""
    B, L, d, bs = 1, 256, 8, 32
    u = np.zeros(d)
    u[2] = 1.0
    q = po.rne(0.1 * np.random.default_rng(13).standard_normal((B, 1, L, d)) + u, "bf16")
    k = 0.1 * np.random.default_rng(14).standard_normal((B, 1, L, d))
    for j in (1, 4):
        k[0, 0, j * bs:(j + 1) * bs] += 3 * u
    k = po.rne(k, "bf16")
    P = m.Problem(B=1, Hq=1, Hkv=1, L=L, d=d, block=bs, topk=2, taylor="order1")
    r = m.run(q, k, _rand((B, 1, L, d), 15, "bf16"), P)
    return all(r["idx"][0, 0, i].tolist() == [1, 4] for i in range(P.n_blk))


def check_pivot_mean(m):
    """The proxy is the mean of its group: members e0 and e1 each prefer a block
    aligned with themselves, their mean prefers the block along e0 + e1."""
    L, d, bs = 64, 8, 8
    q = np.zeros((1, 1, L, d))
    k = np.zeros((1, 1, L, d))
    q[0, 0, 56, 0] = 1.0
    q[0, 0, 57, 1] = 1.0
    k[0, 0, 1 * bs:2 * bs, 0] = 1.0
    k[0, 0, 2 * bs:3 * bs, 1] = 1.0
    k[0, 0, 3 * bs:4 * bs, :2] = 0.75
    P = m.Problem(B=1, Hq=1, Hkv=1, L=L, d=d, dtype="bf16", block=bs, topk=1, group=2,
                  n_cand=1, causal=True, taylor="none")
    r = m.run(q, k, np.ones_like(k), P)
    return r["idx"][0, 0, 56].tolist() == [3] and r["idx"][0, 0, 57].tolist() == [3]


def check_hybrid(m):
    """Hbar by the uncentred identity, and the hybrid output as the order-1
    output averaged over cyclic relabelings of the blocks' H."""
    B, H, L, d, bs = 1, 2, 70, 8, 10
    q, k, v = _rand((B, H, L, d), 16), _rand((B, H, L, d), 17, scale=2.0) + 1.0, _rand((B, H, L, d), 18)
    kw = dict(B=B, Hq=H, Hkv=H, L=L, d=d, dtype="f32", block=bs, topk=2, causal=False)
    Ph, P1 = m.Problem(taylor="hybrid", **kw), m.Problem(taylor="order1", **kw)
    st = m.block_stats(q, k, v, Ph)
    raw = np.einsum("bhsc,bhse->bhce", k, v) - np.einsum("bhjc,bhje->bhce", st["kbar"], st["vsum"])
    ok = np.abs(st["Hbar"] - raw / Ph.n_blk).max() < 1e-11
    idx, _ = m.select(q, st, Ph)
    oh, _ = m.attention(q, k, v, st, idx, Ph)
    acc = sum(m.attention(q, k, v, dict(st, H=np.roll(st["H"], s, axis=2)), idx, P1)[0]
              for s in range(Ph.n_blk)) / Ph.n_blk
    return ok and np.abs(oh - acc).max() < 1e-12


def check_sinks(m):
    """One-token blocks, no top-k: the kept set is the first `sink` tokens and
    the window; and a sink does not take a place in the top-k."""
    B, H, L, d = 1, 1, 30, 6
    q, k, v = _rand((B, H, L, d), 19), _rand((B, H, L, d), 20), _rand((B, H, L, d), 21)
    P = m.Problem(B=B, Hq=H, Hkv=H, L=L, d=d, dtype="f32", block=1, topk=0, window=4, causal=True,
                  taylor="none", sink=3)
    t, s_ = np.arange(L)[:, None], np.arange(L)[None, :]
    mask = (s_ <= t) & ((t - s_ < 4) | (s_ < 3))
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=torch.from_numpy(mask),
        scale=P.sm_scale).numpy()
    ok = np.abs(m.run(q, k, v, P)["O"] - o).max() < 1e-12
    P2 = m.Problem(B=B, Hq=H, Hkv=H, L=L, d=d, dtype="f32", block=1, topk=2, window=4, causal=True,
                   taylor="none", sink=3)
    r = m.run(q, k, v, P2)
    row = r["idx"][0, 0, L - 1]
    return ok and row[:3].tolist() == [0, 1, 2] and (row[3:] >= 3).all() and len(set(row.tolist())) == 5


def check_routing(m):
    """Equal attention scores, closed-form covariance norms (see the pins):
    routing keeps the blocks farthest from the mean first-order matrix, at
    the proxy and at the member stage."""
    nb, bs, d = 8, 8, 8
    a = np.array([0.5, 3.0, -1.0, 2.0, 0.0, 4.0, 1.0, -2.0])
    u, w, c = np.zeros(d), np.zeros(d), np.zeros(d)
    u[1], u[2], w[0], w[3], c[4] = 1.0, 2.0, 1.0, -1.0, 0.5
    e = np.array([1.0, -1.0] * (bs // 2))
    k = (c + (a[:, None] * e[None, :])[:, :, None] * u).reshape(1, 1, nb * bs, d)
    v = (e[None, :, None] * w + 0.25).repeat(nb, axis=0).reshape(1, 1, nb * bs, d)
    q = _rand((1, 1, nb * bs, d), 22, scale=0.3)
    ok = True
    for extra in (dict(), dict(group=4, n_cand=5)):
        P = m.Problem(B=1, Hq=1, Hkv=1, L=nb * bs, d=d, dtype="f32", block=bs, topk=3, taylor="order1",
                      route_lambda=0.5, **extra)
        r = m.run(q, k, v, P)
        ok &= all(r["idx"][0, 0, i].tolist() == [1, 5, 7] for i in range(r["idx"].shape[2]))
    return ok


def check_causal(m):
    """Editing keys and values after position c changes nothing at or before c
    (outputs, lse, selection rows, decode), in the hybrid and first orders, for
    block rows and PIVOT rows; a causal problem with routing is refused."""
    B, Hq, Hkv, L, d, bs = 1, 2, 1, 64, 6, 8
    q, k, v = _rand((B, Hq, L, d), 26, "bf16"), _rand((B, Hkv, L, d), 27, "bf16"), _rand((B, Hkv, L, d), 28, "bf16")
    c = 37
    k2, v2 = k.copy(), v.copy()
    k2[:, :, c + 1:] = _rand(k2[:, :, c + 1:].shape, 29, "bf16", 3.0) + 1.0
    v2[:, :, c + 1:] = _rand(v2[:, :, c + 1:].shape, 30, "bf16", 3.0) - 1.0
    ok = True
    for taylor, extra in (("hybrid", dict(window=12)), ("hybrid", dict(group=2, n_cand=3)),
                          ("order1", dict(window=12))):
        P = m.Problem(B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, block=bs, topk=1, causal=True, taylor=taylor, **extra)
        r, r2 = m.run(q, k, v, P), m.run(q, k2, v2, P)
        ok &= np.abs(r["O"][:, :, :c + 1] - r2["O"][:, :, :c + 1]).max() < 1e-13
        ok &= np.abs(r["lse"][:, :, :c + 1] - r2["lse"][:, :, :c + 1]).max() < 1e-13
        for pos in (c, 20):
            i1 = m.decode_select(q[:, :, pos], r["stats"], P, pos)
            o1, _ = m.decode_attend(q[:, :, pos], k, v, r["stats"], i1, P, pos)
            o2, _ = m.decode_attend(q[:, :, pos], k2, v2, r2["stats"], i1, P, pos)
            ok &= np.abs(o1 - o2).max() < 1e-13
    try:
        m.Problem(B=1, Hq=1, Hkv=1, L=16, d=4, block=4, topk=1, causal=True, route_lambda=0.5)
        ok = False
    except ValueError:
        pass
    return ok


def check_decode(m):
    """The decode step equals the prefill's causal token row at the same position."""
    B, Hq, Hkv, L, d, bs = 1, 2, 1, 40, 6, 8
    q, k, v = _rand((B, Hq, L, d), 23, "bf16"), _rand((B, Hkv, L, d), 24, "bf16"), _rand((B, Hkv, L, d), 25, "bf16")
    ok = True
    for taylor in ("order1", "hybrid"):
        P = m.Problem(B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, block=bs, topk=1, window=10, group=1, n_cand=8,
                      causal=True, taylor=taylor)
        r = m.run(q, k, v, P)
        for pos in (5, 27, 39):
            idx = m.decode_select(q[:, :, pos], r["stats"], P, pos)
            o, _ = m.decode_attend(q[:, :, pos], k, v, r["stats"], idx, P, pos)
            ok &= np.array_equal(idx, r["idx"][:, :, pos]) and np.abs(o - r["O"][:, :, pos]).max() < 1e-12
    return ok


CHECKS = [check_pivot_mean, check_swa_count, check_dense, check_constant_v, check_orders, check_ties,
          check_pivot_reuse, check_pooled_selection, check_hybrid, check_sinks, check_routing, check_decode,
          check_causal]

MUTATIONS = {
    "H transposed": ('H[:, :, j] = np.einsum("bhnc,bhne->bhce", kc, vj)',
                     'H[:, :, j] = np.einsum("bhnc,bhne->bhec", kc, vj)'),
    "first-order sign": ("N = N + sc * np.einsum", "N = N - sc * np.einsum"),
    "first-order without scale": ("N = N + sc * np.einsum", "N = N + 1.0 * np.einsum"),
    "denominator drops n_j": ('pa @ st["n"][Uj].astype(np.float64)', 'pa.sum(axis=1)'),
    "numerator drops sigma": ('+ pa @ st["vsum"][b, hk, Uj]', '+ 0.0'),
    "Taylor logit from ksel": ('a = sc * (qt @ st["kbar"][b, hk, Uj].T)',
                               'a = sc * (qt @ po_round(st["kbar"][b, hk, Uj]).T)'),
    "H not centred": ("kc = kj - kbar[:, :, j][:, :, None, :]", "kc = kj"),
    "window off by one": ("max(0, start - P.window + 1)", "max(0, start - P.window)"),
    "causal mask inclusive bug": ("keys[None, :] <= tt[:, None]", "keys[None, :] < tt[:, None]"),
    "exact ties to higher index": ("ex.sort(reverse=True)", "ex.sort(key=lambda z: (-z[0], z[1]))"),
    "exact ties ranked worst first": ("ex.sort(reverse=True)", "ex.sort()"),
    "GQA head map": ("hk = h * P.Hkv // P.Hq\n    sc = P.sm_scale",
                     "hk = h % P.Hkv\n    sc = P.sm_scale"),
    "proxy is first member": ("qsel[:, :, r] = pooled_mean(q[:, :, r * span:min(L, (r + 1) * span), :], 2, P.dtype)",
                              "qsel[:, :, r] = q[:, :, r * span, :]"),
    "pivot members ignore proxy list": ("tt = top_n(q[b, h, t], Kb[cl], cl, k, bias[cl])",
                                        "tt = top_n(q[b, h, t], Kb[:nc], np.arange(nc), k, bias[:nc])"),
    "hybrid Hbar is the sum": ("Hbar = H.mean(axis=2)", "Hbar = H.sum(axis=2)"),
    "hybrid Hbar over the tail only": ('(qt @ Hb)', '(qt @ st["H"][b, hk, Uj].mean(axis=0))'),
    "hybrid Hbar transposed": ('(qt @ Hb)', '(qt @ Hb.T)'),
    "hybrid term without scale": ('N = N + sc * (qt @ Hb)', 'N = N + 1.0 * (qt @ Hb)'),
    "hybrid causal Hbar over all blocks": ('Hb = st["Hpre"][b, hk, lo] if P.causal else st["Hbar"][b, hk]',
                                           'Hb = st["Hbar"][b, hk]'),
    "hybrid causal prefix takes block lo": ("Hpre[:, :, 1:] = np.cumsum(H, axis=2)[:, :, :-1] / np.arange(1, nb)[:, None, None]",
                                            "Hpre[:, :, 1:] = np.cumsum(H, axis=2)[:, :, 1:] / np.arange(2, nb + 1)[:, None, None]"),
    "routing allowed on causal rows": ("if self.causal and self.route_lambda > 0:", "if False:"),
    "hybrid weights include exact terms": ('* pa.sum(axis=1)[:, None]',
                                           '* (pa.sum(axis=1) + px.sum(axis=1))[:, None]'),
    "sinks take top-k places": ("t = top_n(qsel[b, h, r], Kb[c0:nc], np.arange(c0, nc), k, bias[c0:nc])",
                                "t = top_n(qsel[b, h, r], Kb[:nc], np.arange(nc), k, bias[:nc])[:max(0, k - c0)]"),
    "sinks not kept": ("idx[b, h, r, :c0 + len(t)] = np.concatenate([np.arange(c0), t])",
                       "idx[b, h, r, :len(t)] = t"),
    "routing bias subtracted": ("bias = lam * st[\"M\"][b, hk] if lam > 0", "bias = -lam * st[\"M\"][b, hk] if lam > 0"),
    "routing norm not centred": ("M = np.sqrt(((H - Hbar[:, :, None]) ** 2).sum(axis=(-2, -1)))",
                                 "M = np.sqrt((H ** 2).sum(axis=(-2, -1)))"),
    "routing skipped for members": ("tt = top_n(q[b, h, t], Kb[cl], cl, k, bias[cl])",
                                    "tt = top_n(q[b, h, t], Kb[cl], cl, k)"),
    "decode reads keys past the token": ("np.arange(j * bs, min((j + 1) * bs, pos + 1))", "np.arange(j * bs, (j + 1) * bs)"),
    "decode hybrid term without scale": ('N = N + sc * pa.sum() * (qv @ st["Hpre"][b, hk, lo])',
                                         'N = N + pa.sum() * (qv @ st["Hpre"][b, hk, lo])'),
    "decode hybrid Hbar over all blocks": ('N = N + sc * pa.sum() * (qv @ st["Hpre"][b, hk, lo])',
                                           'N = N + sc * pa.sum() * (qv @ st["Hbar"][b, hk])'),
    "decode window not widened": ("lo = (max(0, pos - P.window + 1) // P.block) if P.window > 0 else own\n    return own, lo, lo",
                                  "lo = (max(0, pos - P.window + 1 + P.block - 1) // P.block) if P.window > 0 else own\n    return own, min(lo, own), min(lo, own)"),
    "scale not applied to exact logits": ("x = sc * (qt @ k[b, hk, keys].T)", "x = (qt @ k[b, hk, keys].T)"),
}


def test_unmodified_oracle_passes_all_checks():
    for c in CHECKS:
        assert c(po), c.__name__


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    src = inspect.getsource(po)
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    src = src.replace(old, new)
    src = src.replace("def rne(", "def po_round(x):\n    return rne(x, 'bf16')\n\n\ndef rne(")
    m = _load(src, f"oracle_mutant_{abs(hash(name))}")
    failed = []
    for c in CHECKS:
        try:
            ok = c(m)
        except Exception:
            ok = False
        if not ok:
            failed.append(c.__name__)
    assert failed, f"no pin check caught the mutation {name!r}"
