"""libpagedattn: paged attention over a block-paged KV cache on MI355X (gfx950).

The compute path is the C-ABI shared library ``libpagedattn.so`` (HIP
kernels plus a host block pool); ``paged_kv_cache_327_amd.binding`` is its
thin ctypes binding.  Importing this package loads nothing; the binding
loads the library on first use and raises if it has not been built.
"""

__all__ = ["binding", "workloads"]
