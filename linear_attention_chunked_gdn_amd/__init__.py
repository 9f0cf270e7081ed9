"""Chunked Gated DeltaNet (gated delta-rule linear attention) for AMD MI355X (gfx950).

The compute lives in a C-ABI HIP library (``libgdn_mi355x.so``, see include/gdn.h);
``gdn`` is its thin Python binding and ``inputs`` holds seeded workload generators.
Nothing is loaded at import time; the first call loads the built library and raises
if it is missing.
"""
from .gdn import GDNError, GDN_BF16, GDN_F32, decode_step, load_library, prefill, prefill_plan

__all__ = ["GDNError", "GDN_BF16", "GDN_F32", "decode_step", "load_library", "prefill",
           "prefill_plan"]
