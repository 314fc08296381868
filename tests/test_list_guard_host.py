"""CPU check of the kept-list guard the kernels apply to caller lists.

The attention and decode kernels keep a list entry j of a selection row only
if 0 <= j < nc, nc the row's candidate count from pisa_row_geometry (the
library's internal header, compiled here for the host with g++).  Reused
lists may hold anything (HyLRA page, section 2.3: tolerant layers attend
with another layer's lists): the guard must keep exactly the entries that
are candidates of the row by the oracle's geometry, drop padding, window-range
blocks, blocks past the row and wild values, and every kept entry must index
inside the kernels' 1024-bit block bitmaps."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import pisa_oracle as po

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "list_guard_probe.cpp")


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path_factory.mktemp("guard") / "guard_probe")
    subprocess.run([gxx, "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "piecewise_attention_dit_amd", "csrc"), SRC, "-o", exe],
                   check=True, capture_output=True)
    return exe


def test_guard_keeps_exactly_the_row_candidates(probe):
    rng = np.random.default_rng(17)
    lines, expect = [], []
    for _ in range(3000):
        bs = int(rng.choice([64, 128]))
        L = int(rng.integers(1, 1024 * bs + 1))
        causal = bool(rng.integers(0, 2))
        window = int(rng.choice([0, 1, 63, 64, 150, 4096])) if causal else 0
        P = po.Problem(B=1, Hq=1, Hkv=1, L=L, d=64, block=bs, topk=4, window=window, causal=causal,
                       group=1 if rng.integers(0, 2) else 0, n_cand=4)
        row = int(rng.integers(0, P.n_rows))
        start = row if P.pivot else row * bs
        own, lo, nc = po.row_geometry(P, row)
        k = int(rng.integers(0, 65))
        wild = [-1, -7, -(2 ** 31), 2 ** 31 - 1, 1024, 1055, 5000, P.n_blk, P.n_blk - 1, own, own + 1,
                (lo if lo is not None else P.n_blk), nc, nc - 1, 0]
        lst = [int(rng.choice(wild)) if rng.random() < 0.4 else int(rng.integers(-3, P.n_blk + 3))
               for _ in range(k)]
        lines.append(f"{L} {bs} {window} {int(causal)} {start} {k} " + " ".join(map(str, lst)))
        expect.append((own, lo if causal else P.n_blk, nc, [j for j in lst if 0 <= j < nc]))
    out = subprocess.run([probe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         check=True).stdout.splitlines()
    assert len(out) == len(expect)
    for got, (own, lo, nc, kept) in zip(out, expect):
        v = [int(x) for x in got.split()]
        assert v[:3] == [own, lo, nc], (got, own, lo, nc)
        assert v[3:] == kept, (got, kept)
        # every kept entry indexes inside the kernels' 32-word block bitmaps
        assert all(0 <= j < 1024 and (j >> 5) < 32 for j in v[3:])
