"""Blockwise-FP8 linear layer for AMD MI355X (gfx950).

The compute path is libfp8blk.so (hand-written HIP kernels behind a C ABI,
declared in include/fp8blk.h).  `binding` exposes the C entry points to Python
with torch tensors for device memory and streams; `linear` wraps the three
GEMMs and the quantisers into an autograd module (Fp8Linear); `workloads` draws
the seeded synthetic inputs; `build` compiles the library.

Importing this package does not load the library; the first call through
`binding` does, and raises if the library is missing.
"""

__all__ = ["binding", "linear", "workloads", "build"]
