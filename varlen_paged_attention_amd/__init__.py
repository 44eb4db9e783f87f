"""varlen_paged_attention_amd: mixed prefill/decode varlen attention over a paged KV
cache, for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libvarlen_attn.so`` built from ``csrc/``; this
package is a thin ctypes binding over its C ABI (``include/varlen_attn.h``).  Importing
the package does not load the library; the first call into ``varlen_paged_attention_amd.api``
does, and raises if it has not been built.
"""
__all__ = ["api", "workloads"]
