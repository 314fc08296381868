"""PISA block-sparse attention for MI355X (gfx950).

The compute path lives in the HIP library ``libpisa.so`` (C ABI declared in
``include/pisa.h``); ``piecewise_attention_dit_amd.pisa`` is its thin ctypes
binding.  Importing this package loads nothing: the library is opened on first
use and a missing or unbuilt library raises an error (there is no fallback).
"""

__all__ = ["pisa", "workloads"]
