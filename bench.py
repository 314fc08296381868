#!/usr/bin/env python3
"""Benchmark of the PISA block-sparse attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input resident in HBM:
pisa_block_stats -> pisa_indexer_topk -> pisa_sparse_attn_fwd.
Prints ONE JSON line.  Default workload: video-DiT self-attention, bf16,
B=1, H=24, L=32760 (21 x 30 x 52 patches), d=128, 128-token blocks, 32 kept
blocks per query block, first-order Taylor for the rest, non-causal.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_F32_VALU_TFLOPS = 256 * 64 * 2 * 2.4e9 / 1e12   # fp32 FMA on the VALU, not packed: 78.6
PEAK_F32_DATASHEET_TFLOPS = 157.3                     # the datasheet's fp32 vector figure (packed fp32)
# source of the attention kernel that runs for block rows (True) / PIVOT rows
ATTN_SRC = {"blocks": os.path.join(ROOT, "piecewise_attention_dit_amd", "csrc", "attn_blocks.hip"),
            "pivot_union": os.path.join(ROOT, "piecewise_attention_dit_amd", "csrc", "attn.hip"),
            "pivot_kg": os.path.join(ROOT, "piecewise_attention_dit_amd", "csrc", "attn_pivot.hip")}


def algorithmic_work(knobs: dict, idx: np.ndarray) -> dict:
    """Algorithmic FLOPs of the attention call and bytes of the stats call,
    from the selections actually made (idx: [B, Hq, n_rows, k], -1 padded).
      exact pairs  (t, s), s in a kept block (s <= t when causal): 4 d FLOPs
      Taylor pairs (t, j), j a non-kept candidate block: 4 d (logit + zero
      order) + 2 d^2 (first order) FLOPs; the hybrid order instead adds
      2 d^2 once per row that has a Taylor block (q Hbar)
      dense-equivalent: 4 d per (t, s) pair of full (causal) attention."""
    B, Hq, Hkv, L, d, bs = (knobs[k] for k in ("B", "Hq", "Hkv", "L", "d", "block"))
    causal, window, group, taylor = knobs["causal"], knobs["window"], knobs["group"], knobs["taylor"]
    n_blk = -(-L // bs)
    nj = np.minimum(bs, L - bs * np.arange(n_blk)).astype(np.int64)
    exact = 0
    taylor_pairs = 0
    taylor_rows = 0
    pivot = group >= 1
    n_rows = idx.shape[2]
    for r in range(n_rows):
        tokens = np.array([r]) if pivot else np.arange(r * bs, min(L, (r + 1) * bs))
        start = r if pivot else r * bs
        own = start // bs
        if causal:
            lo = (max(0, start - window + 1) // bs) if window > 0 else own
            nc = lo
        else:
            lo, nc = n_blk, n_blk
        rows_idx = idx[:, :, r, :]                                      # [B, Hq, k]
        valid = rows_idx >= 0
        kept_keys = np.where(valid, nj[np.clip(rows_idx, 0, n_blk - 1)], 0).sum(axis=-1)  # [B, Hq]
        n_kept = valid.sum(axis=-1)
        if causal:
            win_full = nj[lo:own].sum() if own > lo else 0
            # own block: keys s <= t
            own_pairs = ((tokens - own * bs) + 1).sum()
            exact += int(kept_keys.sum()) * len(tokens) + (win_full * len(tokens) + own_pairs) * B * Hq
        else:
            exact += int(kept_keys.sum()) * len(tokens)
        if taylor != "none":
            taylor_pairs += int((nc - n_kept).sum()) * len(tokens)
            taylor_rows += int((nc - n_kept > 0).sum()) * len(tokens)
    flop_exact = 4 * d * exact
    flop_t0 = 4 * d * taylor_pairs if taylor != "none" else 0
    flop_t1 = (2 * d * d * taylor_pairs if taylor == "order1"
               else 2 * d * d * taylor_rows if taylor == "hybrid" else 0)
    dense_pairs = (L * (L + 1) // 2) if causal else L * L
    dense = 4 * d * dense_pairs * B * Hq
    es = 2 if knobs["dtype"] == "bf16" else 4
    qkv = (B * Hq * L * d + 2 * B * Hkv * L * d) * es
    n_sel = -(-L // group) if pivot else n_blk
    stats_out = B * Hq * n_sel * d * es + B * Hkv * n_blk * d * es
    if taylor != "none":
        stats_out += 2 * B * Hkv * n_blk * d * 4
    if taylor == "order1":
        stats_out += B * Hkv * n_blk * d * d * es
    if taylor == "hybrid":   # one mean matrix, or one per lo for causal rows
        stats_out += B * Hkv * (n_blk if causal else 1) * d * d * es
    return {k: int(v) for k, v in dict(flop_exact=flop_exact, flop_taylor0=flop_t0, flop_taylor1=flop_t1,
                                        flop_attn=flop_exact + flop_t0 + flop_t1, flop_dense=dense,
                                        stats_bytes=qkv + stats_out, exact_pairs=exact,
                                        taylor_pairs=taylor_pairs).items()}


def pivot_executed(knobs: dict, idx: np.ndarray, flop_exact: int) -> dict:
    """Executed MFMA FLOPs of the key-gathered PIVOT kernel and u = executed /
    algorithmic exact FLOPs.  A workgroup pools 256 rows (256 / (Hq / Hkv)
    tokens x the query heads of one kv head); every block one of its rows
    keeps becomes ceil(rows keeping it / 16) tiles per 64-key half, and a tile
    runs 16 rows x 64 keys through S = Q K^T and O = P V (4 d FLOPs a pair)."""
    B, Hq, Hkv, L, d, bs = (knobs[k] for k in ("B", "Hq", "Hkv", "L", "d", "block"))
    causal, window = knobs["causal"], knobs["window"]
    n_blk = -(-L // bs)
    R = Hq // Hkv
    TT = 256 // R
    n_pool = -(-L // TT)
    t = np.arange(L)
    own = t // bs
    if causal:
        lo = (np.maximum(0, t - window + 1) // bs) if window > 0 else own
        nc = lo
    else:
        lo, nc = np.full(L, n_blk), np.full(L, n_blk)
    pool = t // TT
    tiles = 0
    for b in range(B):
        for hk in range(Hkv):
            keys = []
            for h in range(hk * R, hk * R + R):
                lst = np.sort(idx[b, h], axis=1)                         # [L, k]
                ok = (lst >= 0) & (lst < nc[:, None])
                ok[:, 1:] &= lst[:, 1:] != lst[:, :-1]                   # a repeated entry counts once
                keys.append((pool[:, None] * n_blk + lst)[ok])
                if causal:                                               # the range [lo, own]
                    for off in range(int((own - lo).max()) + 1):
                        j = lo + off
                        m = j <= own
                        keys.append(pool[m] * n_blk + j[m])
            cnt = np.bincount(np.concatenate(keys), minlength=n_pool * n_blk)
            tiles += int(((cnt + 15) // 16).sum()) * (bs // 64)
    executed = tiles * 16 * 64 * 4 * d
    return {"tiles": tiles, "flop_executed": executed, "u": round(executed / max(flop_exact, 1), 3)}


def cpu_baseline(wl, q, k, v, budget_s: float) -> dict:
    """The float64 oracle, as it stands, on a bounded sample of the same
    workload: block statistics and selection for query head 0 of batch 0
    (and its KV head), then the attention of that head's query blocks in
    order until the time budget is spent.  The whole-head time is that
    measured time with the attention part scaled to all L rows; the value is
    the head's dense-equivalent FLOPs over it (the metric's unit)."""
    from oracle import pisa_oracle as po

    kn = dict(wl.knobs(), B=1, Hq=1, Hkv=1)
    P = po.Problem.from_knobs(**kn)
    qa, ka, va = (x[:1, :1].double().numpy() for x in (q, k, v))
    t0 = time.perf_counter()
    st = po.block_stats(qa, ka, va, P)
    idx, _ = po.select(qa, st, P)
    t1 = time.perf_counter()
    rows = 0
    step = wl.block if wl.group == 0 else 64
    while rows < wl.L and time.perf_counter() - t1 < budget_s:
        toks = np.arange(rows, min(wl.L, rows + step))
        po.attend_tokens(qa, ka, va, st, idx, P, 0, 0, toks)
        rows += len(toks)
    t2 = time.perf_counter()
    head_time = (t1 - t0) + (t2 - t1) * wl.L / rows
    dense_pairs = (wl.L * (wl.L + 1) // 2) if wl.causal else wl.L * wl.L
    flops = 4 * wl.d * dense_pairs
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    return {"value": round(flops / head_time / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle on query head 0 of batch 0: block stats + selection "
                      f"({t1 - t0:.1f} s), then attention of its first {rows} of {wl.L} rows "
                      f"({t2 - t1:.1f} s), scaled to the whole head; dense-equivalent FLOPs of one head "
                      f"over the scaled time"}


def hbm_traffic(kernel_src: str, workload: str):
    """HBM bytes per launch of the attention kernel from the committed counter
    records (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel
    calibration factor), or None unless a record was taken on this very
    source (sha256) and workload."""
    path = os.path.join(ROOT, "profiles", "attn_traffic.json")
    try:
        with open(path) as f:
            recs = json.load(f).get("records", [])
        with open(kernel_src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    for rec in recs:
        if rec.get("source_sha256") == sha and rec.get("workload") == workload:
            return rec.get("hbm_bytes_per_launch")
    return None


def decode_bench(args):
    """One decode step (decode_topk + decode_fwd) for every (batch, query head)
    of the workload's cache at its last position; one JSON line with the
    token rate and the decode kernel's HBM roofline.  Algorithmic bytes per
    row: keys and values of the exact tokens (kept blocks + window range),
    kbar and vsum of every Taylor block (+ H_j for order 1, + Hbar once for
    the hybrid order), q and o."""
    import torch

    from piecewise_attention_dit_amd import pisa
    from piecewise_attention_dit_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    if args.taylor:
        wl = wl.replace(taylor=args.taylor)
    kn = wl.knobs()
    print(f"[bench] decode: generating the {wl.name} cache", file=sys.stderr, flush=True)
    q, k, v = W.make_inputs(wl)
    p = pisa.make_params(**kn)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    st = pisa.block_stats(p, dq, dk, dv)
    pos = wl.L - 1
    qt = dq[:, :, pos].contiguous()
    idx = pisa.decode_topk(p, pos, qt, st)
    out = torch.empty_like(qt)
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(pisa.workspace_size(p, 3), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        pisa.decode_topk(p, pos, qt, st, idx)
        pisa.decode_fwd(p, pos, qt, dk, dv, st, idx, out=out, lse=lse, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record(stream)
    for _ in range(args.steps):
        pisa.decode_topk(p, pos, qt, st, idx)
    ev[1].record(stream)
    for _ in range(args.steps):
        pisa.decode_fwd(p, pos, qt, dk, dv, st, idx, out=out, lse=lse, ws=ws)
    ev[2].record(stream)
    torch.cuda.synchronize()
    ms_topk = ev[0].elapsed_time(ev[1]) / args.steps
    ms_fwd = ev[1].elapsed_time(ev[2]) / args.steps
    # algorithmic bytes of decode_fwd: per (batch, kv head) the keys and values
    # of the union of its query heads' exact tokens, the statistics of every
    # block that is a Taylor block for one of them, once; q and o per row
    bs, d, es = wl.block, wl.d, (2 if wl.dtype == "bf16" else 4)
    own = pos // bs
    lo = (max(0, pos - wl.window + 1) // bs) if wl.window > 0 else own
    ii = idx.cpu().numpy()
    ratio = wl.Hq // wl.Hkv
    total = 0
    for b in range(wl.B):
        for hk in range(wl.Hkv):
            lists = [set(int(j) for j in ii[b, hk * ratio + r] if 0 <= j < lo) for r in range(ratio)]
            union, common = set().union(*lists), set.intersection(*lists)
            total += (len(union) * bs + (pos + 1 - lo * bs)) * 2 * d * es
            if wl.taylor != "none":
                n_t = lo - len(common)
                total += n_t * 2 * d * 4
                if wl.taylor == "order1":
                    total += n_t * d * d * es
                if wl.taylor == "hybrid":
                    total += d * d * es
    total += wl.B * wl.Hq * 2 * d * es
    per_row = np.array([total])
    gbs = float(per_row.sum()) / (ms_fwd * 1e-3) / 1e9
    rows = wl.B * wl.Hq
    line = {"metric": "decode step: new tokens/s over every (batch, query head) of the cache",
            "value": round(rows / ((ms_topk + ms_fwd) * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_topk + ms_fwd, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
            "data": "synthetic",
            "config": {"workload": f"{wl.name}_decode", "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv,
                       "cache": wl.L, "pos": pos, "d": d, "block": bs, "topk": wl.topk,
                       "window": wl.window, "taylor": wl.taylor},
            "roofline": {"bound": "hbm", "kernel": "pisa_decode_fwd", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": None},
            "kernels": {"decode_topk": {"ms": round(ms_topk, 4)}, "decode_fwd": {"ms": round(ms_fwd, 4),
                        "bytes": int(per_row.sum())}}}
    print(json.dumps(line), flush=True)


def _dist(a) -> dict:
    a = np.asarray(a, dtype=np.float64)
    return {"mean": round(float(a.mean()), 4), "median": round(float(np.median(a)), 4),
            "p10": round(float(np.percentile(a, 10)), 4), "p90": round(float(np.percentile(a, 90)), 4),
            "n": int(a.size)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_peaks(torch, pisa) -> dict:
    """On-box roofline denominators (include/pisa_roofline.h): the best of a
    few runs of the bf16 MFMA loop (1024 workgroups of four waves, four
    independent 32x32x16 chains per wave) and of a 1 GiB HBM copy and read."""
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            work = fn()
            e1.record(stream)
            torch.cuda.synchronize()
            rate = work / (e0.elapsed_time(e1) * 1e-3)
            best = rate if best is None else max(best, rate)
        return best

    wg = 1024
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    pisa.probe_mfma_bf16(wg, 2000, sink)
    mfma = timed(lambda: pisa.probe_mfma_bf16(wg, 60000, sink), 3) / 1e12
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    rsink = torch.zeros(65536, dtype=torch.float32, device="cuda")
    pisa.probe_hbm_copy(dst, src)
    copy = timed(lambda: pisa.probe_hbm_copy(dst, src), 5) / 1e9
    read = timed(lambda: pisa.probe_hbm_read(src, rsink), 5) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma, 1), "hbm_copy_gbs": round(copy, 1), "hbm_read_gbs": round(read, 1),
            "how": "best of 3 runs of a bf16 MFMA 32x32x16 loop (1024 workgroups x 4 waves x 4 chains) and "
                   "of 5 runs of a 1 GiB copy (read + write bytes) and read (HIP events)"}


def indexer_bytes(knobs: dict, wrote_cand: bool) -> int:
    """Algorithmic HBM bytes of pisa_indexer_topk: the pooled selection vectors
    it scores (and, PIVOT, every member query row) read once, the kept lists
    (and proxy lists if asked for) written once."""
    B, Hq, Hkv, L, d, bs = (knobs[k] for k in ("B", "Hq", "Hkv", "L", "d", "block"))
    es = 2 if knobs["dtype"] == "bf16" else 4
    group = knobs["group"]
    n_blk = -(-L // bs)
    klist = knobs["topk"] + knobs.get("sink", 0)
    n_sel = -(-L // group) if group >= 1 else n_blk
    n_rows = L if group >= 1 else n_blk
    total = B * Hq * n_sel * d * es + B * Hkv * n_blk * d * es + B * Hq * n_rows * klist * 4
    if group >= 1:
        total += B * Hq * L * d * es
        if wrote_cand:
            total += B * Hq * n_sel * knobs["n_cand"] * 4
    if knobs.get("route_lambda", 0.0) > 0:
        total += B * Hkv * n_blk * 4
    return total


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="video_dit")
    ap.add_argument("--mode", default="prefill", choices=["prefill", "decode"],
                    help="decode: one new token per (batch, query head) at the end of the "
                         "workload's sequence, read as a cache")
    ap.add_argument("--taylor", default=None, choices=["none", "order0", "order1", "hybrid"],
                    help="run the workload with another treatment of the non-kept blocks "
                         "(reported as workload <name>_<mode>)")
    ap.add_argument("--topk", type=int, default=None,
                    help="run the workload with another top-k (reported as workload <name>_k<topk>); "
                         "topk >= the block count keeps every block: dense attention through the sparse kernel")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the warm-up and the timed steps (for traces): no distribution, "
                         "cold-cache, peak-probe or diagnostic runs")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run three plain device copies of MIB MiB (reads and writes MIB MiB "
                         "each), to calibrate the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    if args.mode == "decode":
        return decode_bench(args)

    import torch

    from piecewise_attention_dit_amd import pisa
    from piecewise_attention_dit_amd import workloads as W

    wl = W.WORKLOADS[args.workload]
    if args.taylor and args.taylor != wl.taylor:
        wl = wl.replace(name=f"{wl.name}_{args.taylor}", taylor=args.taylor)
    if args.topk is not None and args.topk != wl.topk:
        wl = wl.replace(name=f"{wl.name}_k{args.topk}", topk=args.topk)
    knobs = wl.knobs()
    print(f"[bench] generating {wl.name} inputs", file=sys.stderr, flush=True)
    q, k, v = W.make_inputs(wl)
    p = pisa.make_params(**knobs)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    st = pisa.alloc_stats(p)
    idx, _ = pisa.alloc_index(p)      # the proxy lists (diagnostics) are not asked for
    out = torch.empty_like(dq)
    lse = torch.empty((wl.B, wl.Hq, wl.L), dtype=torch.float32, device="cuda")
    ws_need = pisa.workspace_size(p, 0)
    ws = torch.empty(max(ws_need, 16), dtype=torch.uint8, device="cuda")
    ws_attn_need = pisa.workspace_size(p, 2)   # key-gathered PIVOT: K, V^T in fragment order
    ws_attn = torch.empty(max(ws_attn_need, 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        pisa.block_stats(p, dq, dk, dv, st, ws=ws)
        if ev:
            ev[1].record(stream)
        pisa.indexer_topk(p, dq, st, idx, None, want_cand=False)
        if ev:
            ev[2].record(stream)
        pisa.sparse_attn_fwd(p, dq, dk, dv, st, idx, out, lse, ws=ws_attn)
        if ev:
            ev[3].record(stream)

    def per_call(evs):
        return np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                         for e in evs])

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = per_call(evs)
    ms_stats, ms_idx, ms_attn = per.mean(axis=0)
    ms_step = wall * 1e3 / args.steps

    extras = {}
    if not args.no_extras:
        # the same step N more times, for the spread of each call
        n_dist = max(50, args.steps)
        print(f"[bench] distribution over {n_dist} steps", file=sys.stderr, flush=True)
        evd = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_dist)]
        for i in range(n_dist):
            step(evd[i])
        torch.cuda.synchronize()
        extras["dist"] = per_call(evd)
        # cold cache: 512 MiB written before every step (more than the 256 MB
        # last-level cache and the L2s together)
        print("[bench] cold-cache steps", file=sys.stderr, flush=True)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(12)]
        for i in range(12):
            flush.fill_(i & 255)
            step(evc[i])
        torch.cuda.synchronize()
        extras["cold"] = per_call(evc)
        del flush
        # selection diagnostics (counters slow the call: untimed)
        dg = torch.zeros(16, dtype=torch.int32, device="cuda")
        pisa.indexer_topk(p, dq, st, idx, None, want_cand=False, diag=dg)
        torch.cuda.synchronize()
        dgh = dg.cpu().tolist()
        extras["diag"] = {"rows_selected": dgh[0], "rows_rescored": dgh[1], "rows_or_candidates_exact": dgh[2]}
        print("[bench] roofline probes", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        extras["peaks"] = measured_peaks(torch, pisa)

    idx_host = idx.cpu().numpy()
    work = algorithmic_work(knobs, idx_host)
    # bf16 runs on the matrix cores; the fp32 path is plain fp32 FMA on the
    # VALU (no packed fp32): 256 CUs x 64 lanes x 2 FLOP x 2.4 GHz
    peak_kind, peak = ("mfma", PEAK_BF16_TFLOPS) if wl.dtype == "bf16" else ("alu", PEAK_F32_VALU_TFLOPS)
    tflops_eff = work["flop_dense"] / (ms_step * 1e-3) / 1e12
    attn_achieved = work["flop_attn"] / (ms_attn * 1e-3) / 1e12
    stats_gbs = work["stats_bytes"] / (ms_stats * 1e-3) / 1e9
    idx_bytes = indexer_bytes(knobs, wrote_cand=False)
    idx_gbs = idx_bytes / (ms_idx * 1e-3) / 1e9
    kept_frac = work["flop_exact"] / (ms_attn * 1e-3) / 1e12 / peak
    line = {
        "metric": "sparse-attn fwd ms & effective TFLOP/s at L=32K; % of bf16 MFMA / HBM roofline",
        "value": round(tflops_eff, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "L": wl.L, "d": wl.d,
                   "block": wl.block, "topk": wl.topk, "window": wl.window, "group": wl.group,
                   "n_cand": wl.n_cand, "causal": wl.causal, "taylor": wl.taylor,
                   "value_is": "dense-equivalent FLOPs (4 d L^2 B H) / step time"},
        "roofline": {"bound": peak_kind, "kernel": "pisa_sparse_attn_fwd",
                     "achieved": round(attn_achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(attn_achieved / peak, 4),
                     **({} if wl.dtype == "bf16" else
                        {"peak_datasheet": PEAK_F32_DATASHEET_TFLOPS,
                         "peak_note": "the path never forms packed fp32 (v_pk_*_f32), so its peak is the "
                                      "non-packed VALU rate 256 CUs x 64 lanes x 2 FLOP x 2.4 GHz"}),
                     "traffic": hbm_traffic(ATTN_SRC["blocks" if wl.group == 0 else
                                                     "pivot_kg" if ws_attn_need else "pivot_union"], wl.name)
                     if wl.dtype == "bf16" else None},
        "kernels": {
            "block_stats": {"ms": round(ms_stats, 4), "bytes": work["stats_bytes"], "GB/s": round(stats_gbs, 1),
                            "hbm_frac": round(stats_gbs / PEAK_HBM_GBS, 4)},
            "indexer_topk": {"ms": round(ms_idx, 4), "bytes": idx_bytes, "GB/s": round(idx_gbs, 1),
                             "hbm_frac": round(idx_gbs / PEAK_HBM_GBS, 4)},
            "sparse_attn_fwd": {"ms": round(ms_attn, 4),
                                "kept_mfma_frac": round(kept_frac, 4),
                                "total_mfma_frac": round(attn_achieved / peak, 4),
                                "flop_exact": work["flop_exact"], "flop_taylor": work["flop_taylor0"]
                                + work["flop_taylor1"]},
        },
        "host": {"cpu_model": cpu_model(), "cpus": len(os.sched_getaffinity(0))},
    }
    if ws_attn_need:
        line["kernels"]["sparse_attn_fwd"]["executed"] = pivot_executed(knobs, idx_host, work["flop_exact"])
    names = ("block_stats", "indexer_topk", "sparse_attn_fwd")
    if extras:
        for c, nm in enumerate(names):
            line["kernels"][nm]["dist_ms"] = _dist(extras["dist"][:, c])
            line["kernels"][nm]["cold_ms"] = _dist(extras["cold"][:, c])
        line["kernels"]["indexer_topk"].update(extras["diag"])
        pk = extras["peaks"]
        line["measured_peaks"] = pk
        if peak_kind == "mfma":
            line["roofline"]["peak_measured"] = pk["mfma_bf16_tflops"]
            line["roofline"]["frac_measured"] = round(attn_achieved / pk["mfma_bf16_tflops"], 4)
            line["kernels"]["sparse_attn_fwd"]["kept_mfma_frac_measured"] = round(
                kept_frac * peak / pk["mfma_bf16_tflops"], 4)
        for nm, gbs in (("block_stats", stats_gbs), ("indexer_topk", idx_gbs)):
            line["kernels"][nm]["hbm_frac_measured_copy"] = round(gbs / pk["hbm_copy_gbs"], 4)
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, q, k, v, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
