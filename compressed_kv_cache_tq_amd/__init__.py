"""TurboQuant packed KV cache for AMD MI355X (gfx950).

The product is the C-ABI library ``libtq.so`` (HIP kernels for quantization
and decode attention over the packed cache); ``compressed_kv_cache_tq_amd.tq``
is its thin ctypes binding.  ``workloads`` draws the seeded synthetic inputs.
"""
__all__ = ["tq", "workloads"]
