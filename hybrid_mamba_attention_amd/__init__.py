"""MI355X-native H-Spec drafter layer: Mamba-2 state init + SSD scan, and
block-query attention over the target's paged KV cache read in place.

The compute lives in the C-ABI library libhspec.so (hand-written HIP kernels
for gfx950); the Python side only marshals arguments (see `ops`).  Importing
this package does not load the library; the first op call does, and raises if
it is missing.
"""
__all__ = ["workloads", "ops"]
