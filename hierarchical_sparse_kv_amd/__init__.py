"""Hierarchical sparse KV decode attention for MI355X (gfx950).

One decode step: coarse scores of the query against per-thought summary keys,
per-(sequence, KV head) top-k thought selection, then exact softmax attention
over the selected thoughts' tokens plus a recent window, read from a paged
block pool. The work runs in the HIP library ``libzr.so`` (C ABI declared in
include/zr.h); ``hierarchical_sparse_kv_amd.zr`` is its ctypes binding.

Importing the package does not load the library; ``zr.lib()`` does, and raises
if it is missing.
"""
__all__ = ["synth", "zr", "build"]
