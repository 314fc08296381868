"""Vectorised CPU float64 oracle of the PISA block-sparse attention hot path.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  Shares no code with
the HIP library.

Sources (web pages, cited by title and section):
  [PISA]  "PISA: Piecewise Sparse Attention Is Wiser for Efficient Diffusion
          Transformers" (technical summary: section 2 "Methodology" -- core
          algorithm with the N_t / alpha equations, covariance-aware routing,
          hardware implementation).
  [PIVOT] "PIVOT slashes sparse-attention indexer cost 4x ..." (sections "Two
          observations behind PIVOT", steps 1-4, and "Two operating modes").
  [SWA]   "Sliding Window Attention" (glossary; section "How the window widens
          with depth", its code example and printed counts).

The definition implemented (notation of the PISA page):
  * KV blocks of ``bs`` tokens; block j holds tokens [j*bs, min(L,(j+1)*bs)),
    size n_j.  Mean key kbar_j, value sum sigma_j = sum_n v_{j,n} and the
    first-order matrix H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n} (d_k x d_v).
  * Selection vectors are the pooled means rounded to nearest-even into the
    input dtype: qsel (query-block means, or PIVOT proxies = means of g
    consecutive queries) and ksel (key-block means).  Scores are exact real
    dot products qsel . ksel; ties go to the lower block index.
  * Kept set per row r: top-k of its candidate blocks, plus (causal) the
    window/own-block range W_r = [lo_r, own block].
  * Output o_t = N_t / D_t with exact terms over kept tokens and, for every
    non-kept candidate block, alpha = exp(scale q_t . kbar_j) times
    (sigma_j + scale q_t H_j) in N_t and alpha * n_j in D_t (first order per
    block; order 0 drops the H term; "none" drops the block).
  * Attention sinks ([SWA] glossary, attention sinks: StreamingLLM keeps the
    first tokens beside the window): with ``sink`` = s > 0 the first s key
    blocks that are candidates of a row are always kept exactly; the row's
    top-k is chosen among its other candidates, and its kept list holds the
    sink blocks followed by the top-k (width k + s).
  * Covariance-aware routing ([PISA] section 2, covariance-aware routing):
    with route_lambda = lam > 0 a block's selection score is the attention
    score plus lam * M_j, M_j = ||H_j - Hbar|| (Frobenius; the rule that
    combines the two and the weight are not given on the pages: the sum with
    a caller's weight is the reading taken), at every selection stage.  The
    pages define M_j against the global statistic of bidirectional (DiT)
    attention; on causal rows that statistic would carry later tokens, so
    routing is defined for non-causal rows only (a causal problem with
    lam > 0 is refused).
  * Hybrid order ([PISA] section 2, the global first-order correction): zero
    order per non-kept block plus scale q_t Hbar sum_{j in U} alpha_{t,j} in
    N_t, Hbar = the mean of H_j over all blocks of the (batch, KV head).  On a
    causal row, "all blocks" is read as all blocks the row may see as Taylor
    candidates: Hbar_r = the mean of H_j over its candidates [0, lo_r), so no
    statistic of a later token enters the row.
Readings of points the pages leave open are listed in the design notes and
repeated at the functions that take them.
"""
from __future__ import annotations

import dataclasses
import math
from fractions import Fraction

import numpy as np

TAYLOR_MODES = ("none", "order0", "order1", "hybrid")


@dataclasses.dataclass(frozen=True)
class Problem:
    """Problem statement (Q:[B,Hq,L,d], K,V:[B,Hkv,L,d])."""

    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    dtype: str = "bf16"      # "bf16" | "f32": input dtype, also of the pooled vectors
    block: int = 64
    topk: int = 0
    window: int = 0          # causal only
    group: int = 0           # 0: block rows; g >= 1: PIVOT per-token rows, proxies of g
    n_cand: int = 0          # PIVOT proxy list length C
    causal: bool = False
    taylor: str = "order1"
    scale: float = 0.0       # <= 0 -> 1/sqrt(d)
    sink: int = 0            # leading key blocks always kept (attention sinks)
    route_lambda: float = 0.0  # covariance-aware routing weight (0: attention score only)

    def __post_init__(self):
        if self.causal and self.route_lambda > 0:
            raise ValueError("covariance-aware routing is defined for non-causal rows only: its "
                             "global statistic Hbar would carry later tokens into a causal row")

    @property
    def sm_scale(self) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(self.d)

    @property
    def n_blk(self) -> int:
        return -(-self.L // self.block)

    @property
    def pivot(self) -> bool:
        return self.group >= 1

    @property
    def n_rows(self) -> int:
        """Rows of the index list: query blocks, or tokens in PIVOT mode."""
        return self.L if self.pivot else self.n_blk

    @property
    def klist(self) -> int:
        """Width of a kept list: the sink blocks and the top-k."""
        return self.topk + self.sink

    @property
    def n_sel(self) -> int:
        """Rows of the pooled query selection vectors."""
        return -(-self.L // self.group) if self.pivot else self.n_blk

    def block_len(self, j: int) -> int:
        return min(self.block, self.L - j * self.block)

    @classmethod
    def from_knobs(cls, **kw) -> "Problem":
        names = {f.name for f in dataclasses.fields(cls)}
        return cls(**{k: v for k, v in kw.items() if k in names})


# ----------------------------------------------------------------------------
# rounding and exact pooling

_SIG_BITS = {"bf16": 8, "f32": 24}


def rne(x, dtype: str) -> np.ndarray:
    """Round float64 values to nearest, ties to even, into bf16 or fp32 once
    (no intermediate rounding), returned as float64.

    Both formats have an 8-bit exponent (normal exponents -126..127) and p
    significand bits (8 or 24).  The quantum of x is 2^(max(e, -126) - (p-1))
    where 2^e <= |x| < 2^(e+1); x / quantum is rounded half-to-even by
    ``np.rint``; results beyond the largest finite value become +-inf."""
    x = np.asarray(x, dtype=np.float64)
    p = _SIG_BITS[dtype]
    _, e = np.frexp(x)                       # x = m 2^e, 1/2 <= |m| < 1
    qexp = np.maximum(e - 1, -126) - (p - 1)
    y = np.ldexp(np.rint(np.ldexp(x, -qexp)), qexp)
    maxf = (2.0 - 2.0 ** (1 - p)) * 2.0 ** 127
    y = np.where(np.abs(y) > maxf, np.copysign(np.inf, x), y)
    return np.where(np.isfinite(x), y, x)


def exact_sum(x: np.ndarray, axis: int, dtype: str) -> np.ndarray:
    """Correctly rounded float64 sum of dtype values along ``axis``.

    NumPy's float64 sum is exact in any order when every partial sum is an
    integer multiple of the smallest addend quantum 2^emin with magnitude below
    2^(emin+53); that is certified per output from sum|x|.  Outputs that fail
    the certificate are recomputed with ``math.fsum`` (correct rounding)."""
    x = np.asarray(x, dtype=np.float64)
    s = x.sum(axis=axis)
    p = _SIG_BITS[dtype]
    _, e = np.frexp(x)
    lsb = np.where(x != 0, e - p, 10_000)
    emin = lsb.min(axis=axis)
    bound = np.abs(x).sum(axis=axis) * (1.0 + 1e-9)
    ok = (bound < np.ldexp(1.0, np.clip(emin + 52, -1000, 1000))) | (emin >= 10_000)
    if not ok.all():
        xm = np.moveaxis(x, axis, -1)
        for ix in zip(*np.nonzero(~ok)):
            s[ix] = math.fsum(xm[ix].tolist())
    return s


def pooled_mean(x: np.ndarray, axis: int, dtype: str) -> np.ndarray:
    """fl64(fl64(sum) / n): the float64 mean of dtype values (pooling)."""
    n = x.shape[axis]
    return exact_sum(x, axis, dtype) / float(n)


# ----------------------------------------------------------------------------
# stage A: block statistics  ([PISA] section 2, precompute of centroids, value
# sums and first-order matrices; [PIVOT] step 2, proxy = mean of the group)

def block_stats(q: np.ndarray, k: np.ndarray, v: np.ndarray, P: Problem) -> dict:
    """Per KV block: n_j, kbar_j (float64 mean), ksel_j = RNE_dtype(kbar_j),
    sigma_j = sum v, H_j = sum_n (k_n - kbar_j)^T v_n with H_j[c, e] indexed
    (key channel c, value channel e), and Hbar = mean_j H_j over all n_blk
    blocks ([PISA] section 2, the global statistic of the hybrid order; the
    pages average over all blocks, read here as every block of the sequence,
    each with weight 1 / n_blk).  Causal problems also get the prefix table
    Hpre[lo] = mean of H_j over blocks [0, lo) (Hpre[0] = 0), the statistic a
    causal row with candidates [0, lo) uses.  Per query selection row: qsel =
    RNE_dtype(mean of the rows of query block i), or in PIVOT mode the proxy
    RNE_dtype(mean of queries g*gamma .. g*gamma+g-1) (a last partial group
    averages its actual members)."""
    B, Hkv, L, d, bs = P.B, P.Hkv, P.L, P.d, P.block
    nb = P.n_blk
    n = np.array([P.block_len(j) for j in range(nb)], dtype=np.int64)
    kbar = np.empty((B, Hkv, nb, d))
    vsum = np.empty((B, Hkv, nb, d))
    H = np.empty((B, Hkv, nb, d, d))
    for j in range(nb):
        kj = k[:, :, j * bs:j * bs + n[j], :]
        vj = v[:, :, j * bs:j * bs + n[j], :]
        kbar[:, :, j] = pooled_mean(kj, 2, P.dtype)
        vsum[:, :, j] = vj.sum(axis=2)
        kc = kj - kbar[:, :, j][:, :, None, :]
        H[:, :, j] = np.einsum("bhnc,bhne->bhce", kc, vj)
    ksel = rne(kbar, P.dtype)
    span = P.group if P.pivot else bs
    ns = P.n_sel
    qsel = np.empty((B, P.Hq, ns, d))
    for r in range(ns):
        qsel[:, :, r] = pooled_mean(q[:, :, r * span:min(L, (r + 1) * span), :], 2, P.dtype)
    qsel = rne(qsel, P.dtype)
    Hbar = H.mean(axis=2)
    # covariance norm of each block against the mean ([PISA] covariance-aware routing)
    M = np.sqrt(((H - Hbar[:, :, None]) ** 2).sum(axis=(-2, -1)))
    out = dict(n=n, kbar=kbar, ksel=ksel, vsum=vsum, H=H, Hbar=Hbar, M=M, qsel=qsel)
    if P.causal:
        Hpre = np.zeros_like(H)
        Hpre[:, :, 1:] = np.cumsum(H, axis=2)[:, :, :-1] / np.arange(1, nb)[:, None, None]
        out["Hpre"] = Hpre
    return out


# ----------------------------------------------------------------------------
# row geometry ([SWA] causal window 0 <= t - s < w; block rows widen it)

def row_geometry(P: Problem, r: int):
    """(own block, lo, n_cand_blocks) of selection row r.

    Block rows: r is the query block i; its window range is widened to whole
    blocks touching any row's window: lo = blk(max(0, i*bs - w + 1)).
    PIVOT rows: r is the token t; lo = blk(max(0, t - w + 1)).
    Causal: W_r = [lo, own] is kept exactly; candidates are blocks [0, lo).
    Without a window lo = own.  Non-causal: no W_r, candidates are all blocks."""
    start = r if P.pivot else r * P.block
    own = start // P.block
    if not P.causal:
        return own, None, P.n_blk
    lo = (max(0, start - P.window + 1) // P.block) if P.window > 0 else own
    return own, lo, lo


def sink_count(P: Problem, nc: int) -> int:
    """Sink blocks of a row with nc candidates: the first min(s, nc) candidate
    blocks (sinks inside the exact window range are kept by the range)."""
    return min(P.sink, nc)


def group_candidates(P: Problem, gamma: int) -> int:
    """Candidate block count of PIVOT group gamma: the candidates of its first
    member, blocks [0, lo) (a prefix of every member's candidate range)."""
    return row_geometry(P, gamma * P.group)[2]


# ----------------------------------------------------------------------------
# stage B: indexer + top-k ([PISA] covariance-aware routing names the attention
# score; [PIVOT] steps 1-4; block score = pooled dot product)

def exact_score(p: np.ndarray, kv: np.ndarray) -> Fraction:
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(p, kv)), Fraction(0))


def top_n(p: np.ndarray, K: np.ndarray, ids: np.ndarray, n: int, bias=None) -> np.ndarray:
    """The n best of candidates ``ids`` (rows of K) by exact real score
    p.K[j] (+ bias[j], a float64 per candidate), ties to the lower id;
    returned ascending.

    Float64 scores order the candidates; any boundary decision closer than
    1e-12 * (sum|p_c K_jc| + |bias_j|) (far above the float64 error) is
    re-made with exact rational scores."""
    ids = np.asarray(ids)
    m = len(ids)
    if n >= m:
        return np.sort(ids)
    if n <= 0:
        return ids[:0]
    b = np.zeros(m) if bias is None else np.asarray(bias, dtype=np.float64)
    s = K @ p + b
    band = 1e-12 * (np.abs(K) @ np.abs(p) + np.abs(b)) + 1e-300
    order = np.lexsort((ids, -s))
    sel, rest = order[:n], order[n:]
    t_in = (s[sel] - band[sel]).min()
    t_out = (s[rest] + band[rest]).max()
    if t_in > t_out:
        return np.sort(ids[sel])
    amb_sel = sel[s[sel] - band[sel] <= t_out]
    amb_rest = rest[s[rest] + band[rest] >= t_in]
    sure = np.setdiff1d(sel, amb_sel)
    amb = np.concatenate([amb_sel, amb_rest])
    ex = [(exact_score(p, K[a]) + Fraction(float(b[a])), -int(ids[a]), a) for a in amb]
    ex.sort(reverse=True)
    need = n - len(sure)
    chosen = np.array([a for _, _, a in ex[:need]], dtype=np.int64)
    return np.sort(ids[np.concatenate([sure, chosen]).astype(np.int64)])


def select(q: np.ndarray, st: dict, P: Problem):
    """Kept lists.  Returns (idx, cand):
      idx  int64 [B, Hq, n_rows, topk + sink], ascending, -1 padded; row =
           query block (block rows) or token (PIVOT);
      cand int64 [B, Hq, n_groups, n_cand] PIVOT proxy lists (None otherwise).
    With c0 = min(sink, |cand_r|) sink blocks 0 .. c0-1 first, then:
    Block rows: T_r = top-min(k, |cand_r| - c0) of candidates c0 .. by qsel_r . ksel_j.
    PIVOT: Cand_gamma = top-min(C, ..) of the group's candidates past its sinks
    by the proxy's score, then each member t keeps T_t = top-min(k,
    |Cand_gamma|) of Cand_gamma by q_t . ksel_j, after its own sinks (C = k is
    PIVOT-Reuse; g = 1 with C >= |cand| is the dense indexer)."""
    B, Hq, Hkv = P.B, P.Hq, P.Hkv
    k = P.topk
    idx = np.full((B, Hq, P.n_rows, P.klist), -1, dtype=np.int64)
    ksel, qsel = st["ksel"], st["qsel"]
    cand = None
    if P.pivot:
        C = P.n_cand
        ng = P.n_sel
        cand = np.full((B, Hq, ng, C), -1, dtype=np.int64)
    lam = float(np.float32(P.route_lambda))
    for b in range(B):
        for h in range(Hq):
            hk = h * Hkv // Hq
            Kb = ksel[b, hk]
            # covariance-aware routing: lam * M_j added at every selection stage
            bias = lam * st["M"][b, hk] if lam > 0 else np.zeros(P.n_blk)
            if not P.pivot:
                for r in range(P.n_rows):
                    nc = row_geometry(P, r)[2]
                    c0 = sink_count(P, nc)
                    t = top_n(qsel[b, h, r], Kb[c0:nc], np.arange(c0, nc), k, bias[c0:nc])
                    idx[b, h, r, :c0 + len(t)] = np.concatenate([np.arange(c0), t])
            else:
                for gm in range(P.n_sel):
                    nc = group_candidates(P, gm)
                    c0 = sink_count(P, nc)
                    cl = top_n(qsel[b, h, gm], Kb[c0:nc], np.arange(c0, nc), C, bias[c0:nc])
                    cand[b, h, gm, :len(cl)] = cl
                    for t in range(gm * P.group, min(P.L, (gm + 1) * P.group)):
                        ct = sink_count(P, row_geometry(P, t)[2])
                        tt = top_n(q[b, h, t], Kb[cl], cl, k, bias[cl])
                        idx[b, h, t, :ct + len(tt)] = np.concatenate([np.arange(ct), tt])
    return idx, cand


# ----------------------------------------------------------------------------
# stage C: exact + first-order Taylor attention ([PISA] section 2, N_t/D_t
# with the approximations inside both numerator and denominator)

def row_sets(P: Problem, idx_row: np.ndarray, r: int):
    """(kept blocks T_r u W_r, Taylor blocks U_r) of selection row r."""
    own, lo, nc = row_geometry(P, r)
    T = [int(j) for j in idx_row if j >= 0]
    if P.causal:
        kept = sorted(set(T) | set(range(lo, own + 1)))
    else:
        kept = sorted(T)
    U = [] if P.taylor == "none" else sorted(set(range(nc)) - set(T))
    return kept, U


def attend_tokens(q, k, v, st, idx, P: Problem, b: int, h: int, tokens) -> tuple:
    """o_t and lse_t (float64) for the given tokens of (b, query head h).

      m   = max(max_{s in E_t} x_s, max_{j in U_t} a_j),  x_s = scale q.k_s,
                                                         a_j = scale q.kbar_j
      D_t = sum_E e^{x-m} + sum_U e^{a-m} n_j
      N_t = sum_E e^{x-m} v_s + sum_U e^{a-m} (sigma_j + [order1] scale q H_j)
            + [hybrid] scale (q Hbar) sum_U e^{a-m}
      o_t = N_t / D_t,  lse_t = m + ln D_t
    E_t: tokens of kept blocks (s <= t when causal); U_t: Taylor blocks.
    Hbar: over all blocks (non-causal), or over the row's candidates
    [0, lo) (causal)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    hk = h * P.Hkv // P.Hq
    sc = P.sm_scale
    bs = P.block
    out = np.empty((len(tokens), P.d))
    lse = np.empty(len(tokens))
    rows = tokens if P.pivot else tokens // bs
    for r in np.unique(rows):
        sel = np.nonzero(rows == r)[0]
        tt = tokens[sel]
        kept, U = row_sets(P, idx[b, h, r], int(r))
        lo = row_geometry(P, int(r))[1]
        keys = np.concatenate([np.arange(j * bs, j * bs + P.block_len(j)) for j in kept]) \
            if kept else np.zeros(0, dtype=np.int64)
        qt = q[b, h, tt]                                   # [n, d]
        x = sc * (qt @ k[b, hk, keys].T)                   # [n, |E|]
        if P.causal:
            x = np.where(keys[None, :] <= tt[:, None], x, -np.inf)
        Uj = np.asarray(U, dtype=np.int64)
        a = sc * (qt @ st["kbar"][b, hk, Uj].T)            # [n, |U|]
        m = np.maximum(x.max(axis=1, initial=-np.inf), a.max(axis=1, initial=-np.inf))
        px = np.exp(x - m[:, None])
        pa = np.exp(a - m[:, None])
        D = px.sum(axis=1) + pa @ st["n"][Uj].astype(np.float64)
        N = px @ v[b, hk, keys] + pa @ st["vsum"][b, hk, Uj]
        if P.taylor == "order1" and len(Uj):
            qH = np.einsum("nc,jce->nje", qt, st["H"][b, hk, Uj])
            N = N + sc * np.einsum("nj,nje->ne", pa, qH)
        if P.taylor == "hybrid" and len(Uj):
            # causal rows: the mean over the row's candidate blocks [0, lo)
            Hb = st["Hpre"][b, hk, lo] if P.causal else st["Hbar"][b, hk]
            N = N + sc * (qt @ Hb) * pa.sum(axis=1)[:, None]
        out[sel] = N / D[:, None]
        lse[sel] = m + np.log(D)
    return out, lse


def attention(q, k, v, st, idx, P: Problem):
    """Full output [B,Hq,L,d] and lse [B,Hq,L]."""
    O = np.empty((P.B, P.Hq, P.L, P.d))
    lse = np.empty((P.B, P.Hq, P.L))
    allt = np.arange(P.L)
    for b in range(P.B):
        for h in range(P.Hq):
            O[b, h], lse[b, h] = attend_tokens(q, k, v, st, idx, P, b, h, allt)
    return O, lse


def run(q, k, v, P: Problem):
    """Whole path: stats -> selection -> attention.  Inputs are float64 arrays
    holding the dtype values the GPU receives."""
    st = block_stats(q, k, v, P)
    idx, cand = select(q, st, P)
    O, lse = attention(q, k, v, st, idx, P)
    return dict(stats=st, idx=idx, cand=cand, O=O, lse=lse)


# ----------------------------------------------------------------------------
# decode: one new token against a key/value cache ([HyLRA] section 2.3, hybrid
# inference: sensitive layers select the top-k blocks, tolerant layers reuse
# the lists of an earlier layer and attend to that part of the cache only;
# [SWA] the w-slot ring buffer, position i in slot i mod w)

def decode_geometry(P: Problem, pos: int):
    """(own block, lo, number of candidates) of the token at position pos: the
    causal token row of the prefill path (window widened to whole blocks)."""
    own = pos // P.block
    lo = (max(0, pos - P.window + 1) // P.block) if P.window > 0 else own
    return own, lo, lo


def decode_select(q: np.ndarray, st: dict, P: Problem, pos: int) -> np.ndarray:
    """Kept list [B, Hq, topk + sink] of the new token q [B, Hq, d]: the sink
    blocks, then the top-k of the other candidates by the exact score
    q . ksel_j (+ lam M_j with routing), ties to the lower block."""
    B, Hq = q.shape[:2]
    own, lo, nc = decode_geometry(P, pos)
    c0 = min(P.sink, nc)
    lam = float(np.float32(P.route_lambda))
    idx = np.full((B, Hq, P.klist), -1, dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            hk = h * P.Hkv // P.Hq
            bias = lam * st["M"][b, hk, c0:nc] if lam > 0 else None
            t = top_n(q[b, h], st["ksel"][b, hk, c0:nc], np.arange(c0, nc), P.topk, bias)
            idx[b, h, :c0 + len(t)] = np.concatenate([np.arange(c0), t])
    return idx


def decode_attend(q, k, v, st, idx, P: Problem, pos: int) -> tuple:
    """o [B, Hq, d] and lse [B, Hq] of the token at position pos (keys 0..pos
    of the cache k, v [B, Hkv, >= pos + 1, d]) with the kept lists idx
    [B, Hq, >= 1] (-1 padded; from decode_select or reused from another
    layer).  PISA page, section 2: exact terms over the kept blocks and the
    window range [lo, own] (keys s <= pos), Taylor terms for the other
    candidates [0, lo): alpha = e^{scale q . kbar_j} times (sigma_j + [order1]
    scale q H_j) in N and alpha n_j in D, [hybrid] + scale (q Hbar_lo) sum
    alpha with Hbar_lo the mean of H_j over the candidates [0, lo)."""
    B, Hq, d = q.shape
    sc, bs = P.sm_scale, P.block
    own, lo, nc = decode_geometry(P, pos)
    O = np.empty((B, Hq, d))
    lse = np.empty((B, Hq))
    for b in range(B):
        for h in range(Hq):
            hk = h * P.Hkv // P.Hq
            T = sorted(int(j) for j in idx[b, h] if j >= 0)
            kept = sorted(set(T) | set(range(lo, own + 1)))
            keys = np.concatenate([np.arange(j * bs, min((j + 1) * bs, pos + 1)) for j in kept])
            U = [] if P.taylor == "none" else [j for j in range(nc) if j not in set(T)]
            qv = q[b, h]
            x = sc * (k[b, hk, keys] @ qv)
            a = sc * (st["kbar"][b, hk, U] @ qv) if U else np.zeros(0)
            m = max(x.max(), a.max() if len(a) else -np.inf)
            px, pa = np.exp(x - m), np.exp(a - m)
            n_j = np.array([min(bs, P.L - j * bs) for j in U], dtype=np.float64)
            D = px.sum() + pa @ n_j
            N = px @ v[b, hk, keys]
            if U:
                N = N + pa @ st["vsum"][b, hk, U]
                if P.taylor == "order1":
                    N = N + sc * pa @ np.einsum("c,jce->je", qv, st["H"][b, hk, U])
                if P.taylor == "hybrid":
                    N = N + sc * pa.sum() * (qv @ st["Hpre"][b, hk, lo])
            O[b, h] = N / D
            lse[b, h] = m + math.log(D)
    return O, lse


def decode_ring(q, kr, vr, P: Problem, pos: int, w: int) -> tuple:
    """Sliding-window decode from a w-slot ring ([SWA]: token i in slot
    i mod w): the new token at pos attends to tokens max(0, pos - w + 1) ..
    pos exactly.  kr, vr [B, Hkv, w, d]."""
    B, Hq, d = q.shape
    toks = np.arange(max(0, pos - w + 1), pos + 1)
    O = np.empty((B, Hq, d))
    lse = np.empty((B, Hq))
    for b in range(B):
        for h in range(Hq):
            hk = h * P.Hkv // P.Hq
            x = P.sm_scale * (kr[b, hk, toks % w] @ q[b, h])
            m = x.max()
            p = np.exp(x - m)
            O[b, h] = (p @ vr[b, hk, toks % w]) / p.sum()
            lse[b, h] = m + math.log(p.sum())
    return O, lse


# ----------------------------------------------------------------------------
# helpers used by pins and diagnostics

def kept_pairs(P: Problem, idx: np.ndarray, b: int = 0, h: int = 0) -> np.ndarray:
    """Boolean [L, L] matrix of exactly attended (t, s) pairs of one head."""
    M = np.zeros((P.L, P.L), dtype=bool)
    bs = P.block
    for t in range(P.L):
        r = t if P.pivot else t // bs
        kept, _ = row_sets(P, idx[b, h, r], r)
        for j in kept:
            lo, hi = j * bs, j * bs + P.block_len(j)
            M[t, lo:hi] = True
        if P.causal:
            M[t, t + 1:] = False
    return M


def scored_pairs_indexer(P: Problem) -> int:
    """Number of (row, candidate block) dot products the indexer evaluates per
    (b, query head): proxy rows over their candidates plus members over C."""
    if not P.pivot:
        return sum(row_geometry(P, r)[2] for r in range(P.n_rows))
    tot = 0
    for gm in range(P.n_sel):
        nc = group_candidates(P, gm)
        members = min(P.L, (gm + 1) * P.group) - gm * P.group
        tot += nc + members * min(P.n_cand, nc)
    return tot


def dense_indexer_pairs(P: Problem) -> int:
    """Per-token dense indexer cost: every token against all its candidates."""
    return sum(row_geometry(P.__class__(**{**dataclasses.asdict(P), "group": 1}), t)[2]
               for t in range(P.L))
