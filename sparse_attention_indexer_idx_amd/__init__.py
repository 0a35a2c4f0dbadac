"""MI355X-native lightning-indexer hot path: paged MXFP4 K-cache store, MQA scorer and
per-row top-k, as HIP kernels for gfx950 behind a C ABI (``include/idx.h``).

The ctypes binding in ``binding`` carries the C entry points' names; it only marshals
arguments (device pointers, sizes, the current stream).  Importing this package does
not load the HIP library; the first binding call does, and raises if it is missing.
"""
__all__ = ["binding", "workloads"]
