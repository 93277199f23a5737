"""kv_reuse_amd — HySparse2 Cross-Decoder attention (full layer + token top-k + KV-reusing
sparse layers) for AMD Instinct MI355X (gfx950).

The compute lives in ``libhs2.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/hs2.h``).  ``kv_reuse_amd.hs2`` is the thin ctypes
binding; ``kv_reuse_amd.workloads`` builds seeded synthetic inputs.  Importing
this package does not load the library; ``kv_reuse_amd.hs2`` does, and raises
if it has not been built.
"""
__all__ = ["hs2", "workloads"]
