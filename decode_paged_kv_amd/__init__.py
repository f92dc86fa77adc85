"""Paged-KV GQA attention, KV relayout and PD multiplexing on MI355X (gfx950).

The compute path is the HIP library ``libpkv.so`` built from ``csrc/``; the
Python modules here only marshal arguments into its C ABI.  The library is
loaded on first use, and a call fails with ``PkvLibraryMissing`` when it has
not been built: there is no CPU fallback.
"""

__all__ = ["inputs", "workloads"]
