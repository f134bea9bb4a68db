"""Batch-invariant GEMM family and RMSNorm for AMD MI355X (gfx950).

The operations run in hand-written HIP kernels inside ``libbi.so`` behind a
C ABI (``include/bi.h``); ``binding`` only marshals arguments to it, under the
same names (``bi_gemm``, ``bi_bmm``, ``bi_nvfp4_gemm``, ``bi_nvfp4_quant``,
``bi_grouped_gemm``, ``bi_rmsnorm``, ``bi_reduce_rmsnorm``, ``bi_mla_decode``).  The
binding is imported on first use and raises if the library is missing: there
is no CPU fallback.  ``inputs`` (seeded synthetic inputs, NVFP4 host
quantiser) does not need the library.
"""

_BINDING_NAMES = {
    "bi_gemm", "bi_bmm", "bi_nvfp4_gemm", "bi_nvfp4_quant", "bi_grouped_gemm", "bi_rmsnorm",
    "bi_reduce_rmsnorm", "bi_mla_decode", "plan_query", "status_str", "version", "BiError", "lib",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
