"""ShadowKV sparse decode step for MI355X (gfx950).

The decode step of the review page "ShadowKV: KV Cache in Shadows for
High-Throughput Long-Context LLM Inference" (section 三, Algorithms 1-2) as
hand-written HIP kernels behind the C ABI of include/shadowkv.h
(libshadowkv.so).  ``binding`` marshals torch tensors into that ABI,
``setup`` computes the low-rank key factors once per sequence, ``synth``
draws the seeded synthetic workloads.  Nothing is loaded at import time.
"""
__all__ = ["binding", "setup", "synth", "build"]
