"""Gated delta-rule (Gated DeltaNet) sequence mixer for AMD Instinct MI355X.

Chunked prefill and single-token recurrent decode, implemented as gfx950 HIP
kernels behind the C ABI in include/gdn.h.  This package holds the thin
ctypes binding (``gdn``), the seeded synthetic workload generators (``synth``)
and the kernel sources (``csrc``).
"""
from .gdn import (  # noqa: F401
    Context,
    GdnError,
    chunk_prefill,
    chunk_prefill_backward,
    chunk_prefill_frontend,
    decode_step,
    frontend_decode,
    frontend_prefill,
    load_library,
    prefill_backward_workspace_size,
    prefill_workspace_size,
)

__all__ = ["chunk_prefill", "chunk_prefill_frontend", "chunk_prefill_backward", "decode_step", "frontend_prefill", "frontend_decode",
           "prefill_workspace_size", "prefill_backward_workspace_size", "load_library", "GdnError", "Context"]
