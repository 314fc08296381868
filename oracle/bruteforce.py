"""Scalar brute-force re-statement of the PISA hot path (tiny inputs only).

TEST INFRASTRUCTURE ONLY.  Written independently of ``pisa_oracle`` (no shared
helpers) so that the two can be compared: plain Python loops over every
(token, key) and (token, block) pair, pooled means from ``math.fsum``, rounding
to the dtype with exact rationals, and ranking of every candidate by its exact
rational score (ties to the lower block index).

Definition followed: the PISA page, technical summary section 2 (N_t / D_t
with exact terms over selected blocks and, for non-selected blocks,
alpha_{t,j} = exp(q_t . kbar_j) times the block value sum plus the first-order
term, alpha * n_j in the denominator; the hybrid order's global first-order
correction q_t Hbar sum_j alpha_{t,j} with Hbar the mean of the per-block
matrices over all blocks, or, on a causal row, over the blocks it may see as
Taylor candidates, [0, lo)); the PIVOT page's steps 1-4 (proxy =
mean of g consecutive queries, candidates re-ranked per member); the Sliding
Window Attention page's causal mask 0 <= t - s < w, and its attention sinks
(the first blocks of the sequence kept beside the window; the top-k is chosen
among the other candidates); covariance-aware routing adds route_lambda times
the Frobenius norm of H_j - Hbar to every selection score (non-causal rows
only: a causal problem with routing is refused).
"""
from __future__ import annotations

import math
from fractions import Fraction


def _round_frac(x: Fraction, p: int) -> Fraction:
    """Round a rational to p significant bits, ties to even (normal range)."""
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - (p - 1))
    y = a / quantum
    fl = y.numerator // y.denominator
    rem = y - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sgn * fl * quantum


def _pool(rows, dtype):
    """(float64 mean, dtype-rounded mean) of a list of d-vectors."""
    n = len(rows)
    d = len(rows[0])
    mean = [math.fsum(r[c] for r in rows) / n for c in range(d)]
    p = 8 if dtype == "bf16" else 24
    sel = [float(_round_frac(Fraction(x), p)) for x in mean]
    return mean, sel


def run(q, k, v, P):
    """q: nested lists [B][Hq][L][d]; k, v: [B][Hkv][L][d] (Python floats).
    P: an object with the problem fields (B, Hq, Hkv, L, d, dtype, block, topk,
    window, group, n_cand, causal, taylor, sm_scale).  Returns dict with
    'idx' {(b,h,row): sorted kept list}, 'O' {(b,h,t): [d]}, 'lse' {(b,h,t)}."""
    if P.causal and getattr(P, "route_lambda", 0.0) > 0:
        raise ValueError("covariance-aware routing is defined for non-causal rows only")
    bs, L, d = P.block, P.L, P.d
    nb = -(-L // bs)
    blocks = [list(range(j * bs, min(L, (j + 1) * bs))) for j in range(nb)]
    sc = P.sm_scale
    res_idx, res_O, res_lse = {}, {}, {}
    for b in range(P.B):
        for h in range(P.Hq):
            hk = h * P.Hkv // P.Hq
            kb, ks, sg, Hm = [], [], [], []
            for j in range(nb):
                rows = [k[b][hk][s] for s in blocks[j]]
                mean, sel = _pool(rows, P.dtype)
                kb.append(mean)
                ks.append(sel)
                sg.append([sum(v[b][hk][s][e] for s in blocks[j]) for e in range(d)])
                Hm.append([[sum((k[b][hk][s][c] - mean[c]) * v[b][hk][s][e] for s in blocks[j])
                            for e in range(d)] for c in range(d)])

            Hbar = [[sum(Hm[j][c][e] for j in range(nb)) / nb for e in range(d)] for c in range(d)]
            lam = getattr(P, "route_lambda", 0.0)
            Mcov = [math.sqrt(math.fsum((Hm[j][c][e] - Hbar[c][e]) ** 2 for c in range(d) for e in range(d)))
                    for j in range(nb)]

            def geometry(start):
                own = start // bs
                if not P.causal:
                    return own, None, list(range(nb))
                if P.window > 0:
                    lo = max(0, start - P.window + 1) // bs
                else:
                    lo = own
                return own, lo, list(range(lo))

            def rank(pvec, cands, n):
                keyed = []
                for j in cands:
                    ex = sum((Fraction(pvec[c]) * Fraction(ks[j][c]) for c in range(d)), Fraction(0))
                    if lam > 0:
                        ex += Fraction(float(lam) * Mcov[j])
                    keyed.append((-ex, j))
                keyed.sort()
                return sorted(j for _, j in keyed[:n])

            # selection
            kept_of = {}
            sink = getattr(P, "sink", 0)
            if P.group >= 1:
                g = P.group
                for gm in range(-(-L // g)):
                    members = list(range(gm * g, min(L, (gm + 1) * g)))
                    _, proxy = _pool([q[b][h][t] for t in members], P.dtype)
                    _, _, cands = geometry(gm * g)
                    rest = cands[sink:]
                    clist = rank(proxy, rest, min(P.n_cand, len(rest)))
                    for t in members:
                        own_sinks = geometry(t)[2][:sink]
                        kept_of[t] = own_sinks + rank(q[b][h][t], clist, min(P.topk, len(clist)))
                        res_idx[(b, h, t)] = kept_of[t]
            else:
                for i in range(nb):
                    _, qs = _pool([q[b][h][t] for t in blocks[i]], P.dtype)
                    _, _, cands = geometry(i * bs)
                    rest = cands[sink:]
                    kept_of[i] = cands[:sink] + rank(qs, rest, min(P.topk, len(rest)))
                    res_idx[(b, h, i)] = kept_of[i]
            # attention, token by token
            for t in range(L):
                row = t if P.group >= 1 else t // bs
                start = t if P.group >= 1 else (t // bs) * bs
                own, lo, cands = geometry(start)
                T = kept_of[row]
                kept = set(T)
                if P.causal:
                    kept |= set(range(lo, own + 1))
                U = [] if P.taylor == "none" else [j for j in cands if j not in T]
                qt = q[b][h][t]
                terms = []      # (logit, weight in D, numerator vector)
                for j in sorted(kept):
                    for s in blocks[j]:
                        if P.causal and s > t:
                            continue
                        x = sc * sum(qt[c] * k[b][hk][s][c] for c in range(d))
                        terms.append((x, 1.0, list(v[b][hk][s])))
                for j in U:
                    a = sc * sum(qt[c] * kb[j][c] for c in range(d))
                    num = list(sg[j])
                    if P.taylor == "order1":
                        for e in range(d):
                            num[e] += sc * sum(qt[c] * Hm[j][c][e] for c in range(d))
                    terms.append((a, float(len(blocks[j])), num))
                m = max(x for x, _, _ in terms)
                D = sum(math.exp(x - m) * w for x, w, _ in terms)
                N = [sum(math.exp(x - m) * vec[e] for x, _, vec in terms) for e in range(d)]
                if P.taylor == "hybrid" and U:
                    asum = sum(math.exp(sc * sum(qt[c] * kb[j][c] for c in range(d)) - m) for j in U)
                    if P.causal:     # the mean over the row's candidates [0, lo)
                        Hr = [[sum(Hm[j][c][e] for j in range(lo)) / lo for e in range(d)] for c in range(d)]
                    else:
                        Hr = Hbar
                    for e in range(d):
                        N[e] += asum * sc * sum(qt[c] * Hr[c][e] for c in range(d))
                res_O[(b, h, t)] = [N[e] / D for e in range(d)]
                res_lse[(b, h, t)] = m + math.log(D)
    return dict(idx=res_idx, O=res_O, lse=res_lse)
