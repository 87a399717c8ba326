"""Prefix-reuse ("bipartite") attention for generative-recommender prefill on
MI355X (gfx950).

The compute runs in the HIP library ``libbat.so`` (C ABI declared in
``include/bat.h``); ``api`` is the thin torch-tensor binding over it and
``workloads`` draws seeded synthetic inputs.  The library is loaded on first
use and its absence is an error: there is no CPU fallback.
"""
__all__ = ["api", "workloads"]
