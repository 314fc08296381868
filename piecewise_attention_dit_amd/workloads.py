"""Seeded synthetic workloads: shapes, knob values and input generators.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds no part of the attention method's arithmetic: it only
draws Q, K, V with the shapes, value distributions and structure of the
workloads the pages describe (image- and video-DiT self-attention for PISA,
long-context causal LLM prefill for PIVOT and sliding-window attention), and
casts them to the working dtype.

Every generator uses ``numpy.random.default_rng(seed)`` (PCG64), draws in the
fixed order written in its docstring, builds the values in float64, and casts
them to the dtype through float32 (numpy's float64->float32 cast, then torch's
round-to-nearest-even float32->bfloat16).  Both sides of a parity test receive
the very same dtype values.

Tensors are laid out ``[B, H, L, d]``, ``d`` fastest; token order is row-major
over the stated spatial grid.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "PARITY_CASES", "make_inputs", "get"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One problem statement: shapes, sparsity knobs and the input recipe."""

    name: str
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    dtype: str            # "bf16" or "f32"
    block: int            # key/query block size bs
    topk: int             # k blocks per row beyond window / own block
    window: int = 0       # causal sliding window in tokens (0 = none)
    group: int = 0        # 0 = block rows; g >= 1 = PIVOT proxies of g tokens
    n_cand: int = 0       # PIVOT proxy candidate list length C
    causal: bool = False
    taylor: str = "order1"  # "none" | "order0" | "order1" | "hybrid"
    sink: int = 0           # leading key blocks always kept (attention sinks)
    route_lambda: float = 0.0  # covariance-aware routing weight
    recipe: str = "gauss"   # input recipe, see make_inputs
    grid: tuple = ()        # spatial grid (row-major token order) for field recipes
    seed: int = 0

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def knobs(self) -> dict:
        """Problem-statement knobs in the order the C ABI takes them."""
        return dict(B=self.B, Hq=self.Hq, Hkv=self.Hkv, L=self.L, d=self.d,
                    dtype=self.dtype, block=self.block, topk=self.topk,
                    window=self.window, group=self.group, n_cand=self.n_cand,
                    causal=self.causal, taylor=self.taylor, sink=self.sink,
                    route_lambda=self.route_lambda)


# The five headline workloads.  "keep rho" is resolved as k = round(rho * n_blk)
# counting a partial last block (16 of 64, 32 of 256).
WORKLOADS = {
    # Tiny PISA forward, fp32, 32x32 grid with a sinusoidal component.
    "tiny_f32": Workload("tiny_f32", B=1, Hq=2, Hkv=2, L=1024, d=64, dtype="f32",
                         block=64, topk=4, taylor="order1", recipe="sinus",
                         grid=(32, 32)),
    # Image-DiT self-attention, 64x64 latent grid, 2-D blurred shared field.
    "image_dit": Workload("image_dit", B=2, Hq=24, Hkv=24, L=4096, d=64, dtype="bf16",
                          block=64, topk=16, taylor="order1", recipe="field2d",
                          grid=(64, 64)),
    # Video-DiT self-attention, 21 frames x 30 x 52 patches, 3-D blurred field.
    "video_dit": Workload("video_dit", B=1, Hq=24, Hkv=24, L=32760, d=128, dtype="bf16",
                          block=128, topk=32, taylor="order1", recipe="field3d",
                          grid=(21, 30, 52)),
    # Long-context causal LLM prefill with the grouped-proxy (PIVOT) indexer.
    "llm_pivot": Workload("llm_pivot", B=1, Hq=32, Hkv=8, L=65536, d=128, dtype="bf16",
                          block=64, topk=32, group=8, n_cand=128, causal=True,
                          taylor="none", recipe="hot"),
    # Causal sliding window (4096 tokens) + top-16 beyond it, Taylor for the rest.
    "llm_swa": Workload("llm_swa", B=4, Hq=32, Hkv=8, L=32768, d=128, dtype="bf16",
                        block=64, topk=16, window=4096, causal=True, taylor="order1",
                        recipe="ar1"),
}

# Reduced cases the oracle finishes in seconds; each spans several tiles and
# has a ragged tail where the method allows one.
PARITY_CASES = {
    "tiny_f32": WORKLOADS["tiny_f32"],
    "tiny_f32_ragged": WORKLOADS["tiny_f32"].replace(name="tiny_f32_ragged", L=1000,
                                                     grid=(), recipe="gauss", topk=3),
    "image_dit_s": WORKLOADS["image_dit"].replace(name="image_dit_s", B=1, Hq=3, Hkv=3,
                                                  L=1024, grid=(32, 32), topk=4),
    "image_dit_s_o0": WORKLOADS["image_dit"].replace(name="image_dit_s_o0", B=1, Hq=2,
                                                     Hkv=2, L=1024, grid=(32, 32), topk=4,
                                                     taylor="order0"),
    "video_dit_s": WORKLOADS["video_dit"].replace(name="video_dit_s", Hq=2, Hkv=2,
                                                  L=2 * 13 * 40, grid=(2, 13, 40), topk=2),
    "video_dit_s_none": WORKLOADS["video_dit"].replace(name="video_dit_s_none", Hq=2,
                                                       Hkv=2, L=1000, grid=(1, 20, 50),
                                                       topk=3, taylor="none"),
    "llm_pivot_s": WORKLOADS["llm_pivot"].replace(name="llm_pivot_s", Hq=8, Hkv=2,
                                                  L=2048 + 40, topk=6, n_cand=12),
    "llm_pivot_s_reuse": WORKLOADS["llm_pivot"].replace(name="llm_pivot_s_reuse", Hq=4,
                                                        Hkv=1, L=1536, topk=5, n_cand=5),
    "llm_swa_s": WORKLOADS["llm_swa"].replace(name="llm_swa_s", B=1, Hq=8, Hkv=2,
                                              L=2048 + 24, window=384, topk=4),
    "llm_swa_s_b128": WORKLOADS["llm_swa"].replace(name="llm_swa_s_b128", B=1, Hq=4,
                                                   Hkv=1, L=1900, block=128, window=300,
                                                   topk=3, taylor="order0"),
    # hybrid order: every attention kernel and both Hbar kernels
    "tiny_f32_hyb": WORKLOADS["tiny_f32"].replace(name="tiny_f32_hyb", L=1000, grid=(),
                                                  recipe="gauss", topk=3, taylor="hybrid"),
    "image_dit_s_hyb": WORKLOADS["image_dit"].replace(name="image_dit_s_hyb", B=1, Hq=2,
                                                      Hkv=2, L=1024, grid=(32, 32), topk=4,
                                                      taylor="hybrid"),
    "video_dit_s_hyb": WORKLOADS["video_dit"].replace(name="video_dit_s_hyb", Hq=2, Hkv=2,
                                                      L=1000, grid=(1, 20, 50), topk=2,
                                                      taylor="hybrid"),
    "llm_swa_s_hyb": WORKLOADS["llm_swa"].replace(name="llm_swa_s_hyb", B=2, Hq=4, Hkv=2,
                                                  L=2048 + 24, window=384, topk=4,
                                                  taylor="hybrid"),
    "llm_pivot_s_hyb": WORKLOADS["llm_pivot"].replace(name="llm_pivot_s_hyb", Hq=4, Hkv=2,
                                                      L=1024 + 40, topk=4, n_cand=8,
                                                      taylor="hybrid"),
    # zero order / hybrid order over more than two batches of 16 Taylor
    # entries (the staged batch tables run two batches ahead)
    "video_dit_m_o0": WORKLOADS["video_dit"].replace(name="video_dit_m_o0", Hq=2, Hkv=2,
                                                     L=5120, grid=(1, 40, 128), topk=4,
                                                     taylor="order0"),
    "video_dit_m_hyb": WORKLOADS["video_dit"].replace(name="video_dit_m_hyb", Hq=2, Hkv=2,
                                                      L=5120, grid=(1, 40, 128), topk=4,
                                                      taylor="hybrid"),
    "image_dit_m_hyb": WORKLOADS["image_dit"].replace(name="image_dit_m_hyb", B=1, Hq=2,
                                                      Hkv=2, L=4096, grid=(64, 64), topk=8,
                                                      taylor="hybrid"),
    "llm_swa_m_hyb": WORKLOADS["llm_swa"].replace(name="llm_swa_m_hyb", B=1, Hq=4, Hkv=1,
                                                  L=6400 + 24, window=384, topk=4,
                                                  taylor="hybrid"),
    # attention sinks: block-row and PIVOT indexers, every attention kernel
    "llm_swa_s_sink": WORKLOADS["llm_swa"].replace(name="llm_swa_s_sink", B=1, Hq=8, Hkv=2,
                                                   L=2048 + 24, window=384, topk=4, sink=2),
    "llm_pivot_s_sink": WORKLOADS["llm_pivot"].replace(name="llm_pivot_s_sink", Hq=8, Hkv=2,
                                                       L=2048 + 40, topk=6, n_cand=12, sink=2),
    "video_dit_s_sink": WORKLOADS["video_dit"].replace(name="video_dit_s_sink", Hq=2, Hkv=2,
                                                       L=1000, grid=(1, 20, 50), topk=2, sink=1,
                                                       taylor="hybrid"),
    # covariance-aware routing, weights that make both terms of the score count
    # (covariance routing is defined for non-causal rows: the LLM shapes run
    # bidirectional here)
    "gqa_s_route": WORKLOADS["llm_swa"].replace(name="gqa_s_route", B=1, Hq=8, Hkv=2,
                                                L=2048 + 24, window=0, causal=False, topk=4,
                                                route_lambda=0.04),
    "video_dit_s_route": WORKLOADS["video_dit"].replace(name="video_dit_s_route", Hq=2, Hkv=2,
                                                        L=1000, grid=(1, 20, 50), topk=2,
                                                        taylor="hybrid", route_lambda=0.05),
    "pivot_s_route": WORKLOADS["llm_pivot"].replace(name="pivot_s_route", Hq=8, Hkv=2,
                                                    L=2048 + 40, topk=6, n_cand=12, causal=False,
                                                    taylor="order0", route_lambda=0.016),
    # causal hybrid order with a window that spans several blocks per tile
    "llm_swa_s_hyb_w": WORKLOADS["llm_swa"].replace(name="llm_swa_s_hyb_w", B=1, Hq=8, Hkv=8,
                                                    L=2048 + 24, window=200, topk=3,
                                                    taylor="hybrid"),
    "llm_pivot_s_hyb_w": WORKLOADS["llm_pivot"].replace(name="llm_pivot_s_hyb_w", Hq=2, Hkv=2,
                                                        L=1024 + 40, topk=3, n_cand=6, window=150,
                                                        taylor="hybrid"),
}


def get(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    return PARITY_CASES[name]


# ----------------------------------------------------------------------------
# generators

def _to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _gauss(rng, shape):
    return rng.standard_normal(size=shape)


def _sinus(rng, wl: Workload, H: int) -> np.ndarray:
    """N(0,1) + 1.5*sin(2*pi*(fx*x + fy*y)/32 + phi); fx, fy in {1,2} and phi in
    [0, 2pi) drawn per (head, channel).  Draws: noise [B,H,L,d], then fx, fy, phi."""
    gy, gx = wl.grid
    assert gy * gx == wl.L
    noise = rng.standard_normal(size=(wl.B, H, wl.L, wl.d))
    fx = rng.integers(1, 3, size=(H, wl.d))
    fy = rng.integers(1, 3, size=(H, wl.d))
    phi = rng.uniform(0.0, 2.0 * math.pi, size=(H, wl.d))
    y, x = np.divmod(np.arange(wl.L), gx)
    arg = 2.0 * math.pi * (fx[None, :, None, :] * x[None, None, :, None]
                           + fy[None, :, None, :] * y[None, None, :, None]) / 32.0
    return noise + 1.5 * np.sin(arg + phi[None, :, None, :])


def _smooth_field(rng, B, H, d, grid, sigma):
    """I.i.d. N(0,1) on the grid per (b, h, channel), Gaussian blur (reflect,
    truncated at 4 sigma), renormalised to unit standard deviation; returned as
    [B, H, L, d] with row-major token order."""
    from scipy.ndimage import gaussian_filter

    white = rng.standard_normal(size=(B, H, d) + tuple(grid))
    sig = (0, 0, 0) + tuple(sigma)
    f = gaussian_filter(white, sigma=sig, mode="reflect", truncate=4.0)
    axes = tuple(range(3, 3 + len(grid)))
    f = f / f.std(axis=axes, keepdims=True)
    L = int(np.prod(grid))
    return np.moveaxis(f.reshape(B, H, d, L), 2, 3)


def make_inputs(wl: Workload, seed: int | None = None):
    """Return (q, k, v) as CPU torch tensors of the workload's dtype.

    Recipes (draw order in parentheses):
      gauss   Q, K, V ~ N(0,1)                                   (Q, K, V)
      sinus   each of Q, K, V = N(0,1) + 1.5 sin(...)            (Q, K, V; each as _sinus)
      field2d Q, K = 0.5 N(0,1) + F, F a 2-D blurred field (sigma 4 patches)
              shared by Q and K; V ~ N(0,1)                      (Q noise, K noise, V, F)
      field3d Q, K = F + 0.5 N(0,1), F blurred with sigma (1 frame, 3, 3)
              shared by Q and K; V ~ N(0,1)                      (Q noise, K noise, V, F)
      hot     Q, K, V ~ N(0,1); u = N(0,I_d)/|.|; per KV head 64 (or n_blk/16 if
              fewer blocks) distinct hot blocks get +3u on every key
                                                                 (Q, K, V, u, hot blocks)
      ar1     each of Q, K, V = N(0,1) + r, r_t = 0.98 r_{t-1} + sqrt(1-0.98^2) eta_t,
              r_0 ~ N(0,1), independent per (tensor, b, head, channel)
                                                                 (per tensor, per (b, head):
                                                                  noise then eta)
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, Hq, Hkv, L, d = wl.B, wl.Hq, wl.Hkv, wl.L, wl.d
    r = wl.recipe
    if r == "gauss":
        q = _gauss(rng, (B, Hq, L, d))
        k = _gauss(rng, (B, Hkv, L, d))
        v = _gauss(rng, (B, Hkv, L, d))
    elif r == "sinus":
        q = _sinus(rng, wl, Hq)
        k = _sinus(rng, wl, Hkv)
        v = _sinus(rng, wl, Hkv)
    elif r in ("field2d", "field3d"):
        assert Hq == Hkv, "shared-field recipes are for multi-head (Hq == Hkv) layouts"
        nq = rng.standard_normal(size=(B, Hq, L, d))
        nk = rng.standard_normal(size=(B, Hkv, L, d))
        v = rng.standard_normal(size=(B, Hkv, L, d))
        sigma = (4.0, 4.0) if r == "field2d" else (1.0, 3.0, 3.0)
        f = _smooth_field(rng, B, Hq, d, wl.grid, sigma)
        q = 0.5 * nq + f
        k = 0.5 * nk + f
        del nq, nk, f
    elif r == "hot":
        n_blk = -(-L // wl.block)
        n_hot = min(64, max(1, n_blk // 16))
        q = _to_dtype(_gauss(rng, (B, Hq, L, d)), wl.dtype)
        k = _gauss(rng, (B, Hkv, L, d))
        v = _gauss(rng, (B, Hkv, L, d))
        u = rng.standard_normal(size=d)
        u = u / np.linalg.norm(u)
        for b in range(B):
            for h in range(Hkv):
                hot = rng.choice(n_blk, size=n_hot, replace=False)
                for j in hot:
                    k[b, h, j * wl.block:(j + 1) * wl.block, :] += 3.0 * u
        return q, _to_dtype(k, wl.dtype), _to_dtype(v, wl.dtype)
    elif r == "ar1":
        from scipy.signal import lfilter

        rho = 0.98
        c = math.sqrt(1.0 - rho * rho)
        outs = []
        for H in (Hq, Hkv, Hkv):
            t = torch.empty((B, H, L, d), dtype=wl.torch_dtype)
            for b in range(B):
                for h in range(H):
                    noise = rng.standard_normal(size=(L, d))
                    eta = rng.standard_normal(size=(L, d))
                    eta[1:] *= c
                    # the recurrence runs along tokens; filtering the
                    # transposed copy is the same arithmetic, contiguous
                    drift = lfilter([1.0], [1.0, -rho], np.ascontiguousarray(eta.T), axis=-1).T
                    t[b, h] = _to_dtype(noise + drift, wl.dtype)
            outs.append(t)
        return tuple(outs)
    else:
        raise ValueError(f"unknown recipe {r!r}")
    return _to_dtype(q, wl.dtype), _to_dtype(k, wl.dtype), _to_dtype(v, wl.dtype)
