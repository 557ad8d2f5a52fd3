"""MI355X-native HSTU pointwise aggregated attention (gfx950 HIP kernels behind a C ABI).

The compute lives in ``libhstu.so`` (hand-written HIP kernels for gfx950);
this package only marshals arguments to it.  Importing the package does not
load the library; the first call does, and raises if it is missing.
"""
from .flops import attn_flops, visible_pairs  # noqa: F401

__all__ = ["attn_flops", "visible_pairs"]
