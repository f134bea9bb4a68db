"""Batch-invariant GEMM family and RMSNorm for AMD MI355X (gfx950).

The operations run in hand-written HIP kernels inside ``libbi.so`` behind a
C ABI (``include/bi.h``); this package only marshals arguments to it.  The
binding is loaded on first use and raises if the library is missing: there is
no CPU fallback.
"""
