"""block_top_sparse_amd: block top-k sparse decode attention for MI355X (gfx950).

The compute lives in a hand-written HIP library (csrc/, built into
libkin.so) behind a C ABI declared in include/kin.h.  The Python binding in
`binding` only marshals arguments: every step of the path runs in the HIP
kernels, and every call raises if the library is missing.
"""
__all__ = ["binding", "workloads", "synth"]
