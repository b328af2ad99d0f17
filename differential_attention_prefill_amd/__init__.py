"""MI355X-native differential attention: lambda, fused prefill, split-KV decode.

The compute lives in ``libdiffattn.so`` (hand-written HIP for gfx950 behind a
C ABI declared in ``include/diffattn.h``); ``api`` is a thin ctypes binding
with the same entry-point names, and ``workloads`` draws seeded inputs.
"""
__all__ = ["api", "workloads"]
