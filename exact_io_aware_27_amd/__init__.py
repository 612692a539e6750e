"""Exact, fused attention forward pass for AMD MI355X (gfx950).

The product is the C-ABI library ``libattn.so`` (declared in include/attn.h,
built from ``csrc/``).  ``exact_io_aware_27_amd.attn`` is its thin Python
binding; ``exact_io_aware_27_amd.inputs`` draws the seeded synthetic inputs.
Importing the package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""

__all__ = ["attn", "inputs"]
