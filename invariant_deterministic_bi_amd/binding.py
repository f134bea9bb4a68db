"""ctypes binding of libbi (include/bi.h): argument marshalling only.

Each function takes torch tensors (device memory) or raw integers, passes
pointers, strides and the current HIP stream to the C entry point of the same
name, and raises ``BiError`` on a non-zero status.  Every step of the
computation runs in libbi's HIP kernels; if the library is missing this
module raises on load -- there is no fallback.

torch is imported before the library is opened so that libbi binds to the HIP
runtime torch has already loaded (one runtime per process, so torch's
streams and allocations are valid inside libbi).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbi.so")

(BI_OK, BI_ERR_NULL, BI_ERR_SHAPE, BI_ERR_ALIGN, BI_ERR_ALIAS, BI_ERR_UNSUPPORTED, BI_ERR_HIP,
 BI_ERR_VALUE) = range(8)
BI_A_BF16, BI_A_NVFP4 = 0, 1
(BI_OP_GEMM, BI_OP_BMM, BI_OP_NVFP4_GEMM, BI_OP_RMSNORM, BI_OP_NVFP4_QUANT, BI_OP_REDUCE_RMSNORM,
 BI_OP_GROUPED_GEMM) = range(7)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class BiPlan(ctypes.Structure):
    _fields_ = [("op", _i32), ("bm", _i32), ("bn", _i32), ("bk", _i32), ("mfma_m", _i32),
                ("mfma_n", _i32), ("mfma_k", _i32), ("waves", _i32), ("lds_stages", _i32),
                ("threads", _i32), ("chunks_per_thread", _i32), ("reserved", _i32 * 5)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved"}


class BiRegime(ctypes.Structure):
    _fields_ = [("kernel", _i32), ("m_min", _i32), ("m_max", _i32), ("row_blocks", _i32), ("cols", _i32),
                ("a_pairs", _i32), ("a_rows_staged", _i32), ("tile_variant", _i32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


KERNEL_KINDS = ("tiled", "tiled_pingpong", "stream_a_lds", "stream_reg", "stream_ring", "bmm_stream",
                "stream_a_chunks")


class BiLaunchOpts(ctypes.Structure):
    _fields_ = [("max_workgroups", _i32), ("tile_variant", _i32), ("pipeline_depth", _i32),
                ("fixed_plan", _i32), ("reserved", _i32 * 4)]


class BiError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


_lib = None

_SIGS = {
    "bi_gemm": [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p],
    "bi_gemm_ex": [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _p],
    "bi_bmm": [_p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64, _i64, _i64, _i64, _p],
    "bi_bmm_ex": [_p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p],
    "bi_nvfp4_gemm": [_p, _p, ctypes.c_int, _i64, _p, _p, ctypes.c_float, _p, _i64, _i64, _i64,
                      _i64, _p],
    "bi_nvfp4_gemm_ex": [_p, _p, ctypes.c_int, _i64, _p, _p, ctypes.c_float, _p, _i64, _i64,
                         _i64, _i64, _p, _p],
    "bi_rmsnorm": [_p, _i64, _p, ctypes.c_float, _p, _i64, _i64, _i64, _p],
    "bi_rmsnorm_ex": [_p, _i64, _p, ctypes.c_float, _p, _i64, _i64, _i64, _p, _p],
    "bi_nvfp4_quant": [_p, _i64, ctypes.c_float, _p, _p, _i64, _i64, _i64, _p],
    "bi_nvfp4_quant_ex": [_p, _i64, ctypes.c_float, _p, _p, _i64, _i64, _i64, _p, _p],
    "bi_reduce_rmsnorm": [ctypes.POINTER(_p), ctypes.c_int, _i64, _p, _i64, _p, ctypes.c_float, _p,
                          _i64, _p, _i64, _i64, _i64, _p],
    "bi_reduce_rmsnorm_ex": [ctypes.POINTER(_p), ctypes.c_int, _i64, _p, _i64, _p, ctypes.c_float,
                             _p, _i64, _p, _i64, _i64, _i64, _p, _p],
    "bi_grouped_gemm": [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p],
    "bi_grouped_gemm_ex": [_p, _i64, _p, _i64, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _p],
    "bi_mla_decode": [_p, _p, _p, ctypes.c_float, _p, _i64, _i64, _i64, _i64, _i64, _p, _i64, _p],
    "bi_mla_decode_ex": [_p, _p, _p, ctypes.c_float, _p, _i64, _i64, _i64, _i64, _i64, _p, _i64, _p, _p],
    "bi_mla_decode_noalloc": [_p, _p, _p, ctypes.c_float, _p, _i64, _i64, _i64, _i64, _i64, _p],
    "bi_mla_decode_workspace_size": [_i64, _i64, _i64, _i64, _i64, ctypes.POINTER(ctypes.c_int64)],
    "bi_plan_query": [ctypes.c_int, _i64, _i64, ctypes.POINTER(BiPlan)],
    "bi_tile_shape": [ctypes.c_int, ctypes.POINTER(BiPlan)],
    "bi_probe_mfma": [_p, _i64, ctypes.c_int, _p],
    "bi_probe_read": [_p, _i64, _p, ctypes.c_int, _p],
    "bi_probe_lds": [_p, _i64, ctypes.c_int, _p],
    "bi_plan_regimes": [ctypes.c_int, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(BiRegime),
                        ctypes.c_int, ctypes.POINTER(ctypes.c_int)],
}


def lib() -> ctypes.CDLL:
    """The loaded libbi (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libbi.so not found at {LIB_PATH}: build it with "
            "`python -m invariant_deterministic_bi_amd.build` (there is no CPU fallback)")
    l = ctypes.CDLL(LIB_PATH)
    for name, args in _SIGS.items():
        f = getattr(l, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    l.bi_status_str.argtypes = [ctypes.c_int]
    l.bi_status_str.restype = ctypes.c_char_p
    l.bi_version.argtypes = []
    l.bi_version.restype = ctypes.c_char_p
    _lib = l
    return l


def status_str(status: int) -> str:
    return lib().bi_status_str(int(status)).decode()


def version() -> str:
    return lib().bi_version().decode()


def plan_query(op: int, N: int, K: int) -> dict:
    pl = BiPlan()
    st = lib().bi_plan_query(int(op), int(N), int(K), ctypes.byref(pl))
    if st != BI_OK:
        raise BiError(st, "bi_plan_query")
    return pl.as_dict()


def plan_regimes(op: int, N: int, K: int, a_fmt: int = BI_A_BF16, cus: int = 0) -> list:
    """Every kernel an (op, N, K) call can run and the row ranges that select
    it (bi_plan_regimes), as dicts with a 'kind' name added."""
    cap = 64
    arr = (BiRegime * cap)()
    n = ctypes.c_int(0)
    st = lib().bi_plan_regimes(int(op), int(N), int(K), int(a_fmt), int(cus), arr, cap, ctypes.byref(n))
    if st != BI_OK:
        raise BiError(st, "bi_plan_regimes")
    out = []
    for i in range(n.value):
        d = arr[i].as_dict()
        d["kind"] = KERNEL_KINDS[d["kernel"]]
        out.append(d)
    return out


def tile_shapes() -> list:
    """The compiled GEMM tile shapes (index v is tile_variant v+1)."""
    out = []
    v = 0
    while True:
        pl = BiPlan()
        if lib().bi_tile_shape(v, ctypes.byref(pl)) != BI_OK:
            return out
        out.append(pl.as_dict())
        v += 1


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _opts(max_workgroups=0, tile_variant=0, pipeline_depth=0, fixed_plan=False):
    if not max_workgroups and not tile_variant and not pipeline_depth and not fixed_plan:
        return None
    o = BiLaunchOpts()
    o.max_workgroups = int(max_workgroups)
    o.tile_variant = int(tile_variant)
    o.pipeline_depth = int(pipeline_depth)
    o.fixed_plan = 1 if fixed_plan else 0
    return ctypes.byref(o)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check2d(t, name, dtypes=(torch.bfloat16, torch.int16, torch.uint16)):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit stride along the last dimension")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not accepted")


def _raise(st, what):
    if st != BI_OK:
        raise BiError(st, what)


def bi_gemm(A, B, Y=None, *, stream=None, max_workgroups=0, tile_variant=0, pipeline_depth=0, fixed_plan=False):
    """Y[M,N] = A[M,K] . B[N,K]^T (bf16); allocates Y with torch if not given."""
    _check2d(A, "A")
    _check2d(B, "B")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    _check2d(Y, "Y")
    if tuple(Y.shape) != (M, N):
        raise ValueError("Y must be [M, N]")
    st = lib().bi_gemm_ex(_ptr(A), A.stride(0), _ptr(B), B.stride(0), _ptr(Y), Y.stride(0),
                          M, N, K, _stream(stream), _opts(max_workgroups, tile_variant, pipeline_depth, fixed_plan))
    _raise(st, "bi_gemm")
    return Y


def bi_bmm(A, B, Y=None, *, stream=None, max_workgroups=0, tile_variant=0):
    """Y[h] = A[h] . B[h] for A [H,M,K], B [H,K,N] (bf16)."""
    if A.dim() != 3 or B.dim() != 3 or A.stride(2) != 1 or B.stride(2) != 1:
        raise ValueError("A and B must be 3-D with unit stride along the last dimension")
    H, M, K = A.shape
    H2, K2, N = B.shape
    if H != H2 or K != K2:
        raise ValueError("A [H,M,K] and B [H,K,N] disagree")
    if Y is None:
        Y = torch.empty((H, M, N), dtype=torch.bfloat16, device=A.device)
    if tuple(Y.shape) != (H, M, N) or Y.stride(2) != 1:
        raise ValueError("Y must be [H, M, N] with unit last stride")
    st = lib().bi_bmm_ex(_ptr(A), A.stride(0), A.stride(1), _ptr(B), B.stride(0), B.stride(1),
                         _ptr(Y), Y.stride(0), Y.stride(1), H, M, N, K, _stream(stream),
                         _opts(max_workgroups, tile_variant))
    _raise(st, "bi_bmm")
    return Y


def bi_nvfp4_gemm(A, W, W_scales, alpha, Y=None, *, A_scales=None, K=None, stream=None,
                  max_workgroups=0, tile_variant=0, pipeline_depth=0, fixed_plan=False):
    """Y[M,N] = alpha * A . W^T with NVFP4 W (codes [N,K/2] uint8, scales [N,K/16] uint8).

    A is bf16 [M,K] when A_scales is None, else NVFP4 codes [M,K/2] with
    scales [M,K/16].
    """
    N = W.shape[0]
    if K is None:
        K = W.shape[1] * 2
    if tuple(W.shape) != (N, K // 2) or tuple(W_scales.shape) != (N, K // 16):
        raise ValueError("W must be [N,K/2] and W_scales [N,K/16]")
    if not (W.is_contiguous() and W_scales.is_contiguous()):
        raise ValueError("W and W_scales must be dense")
    M = A.shape[0]
    if A_scales is None:
        _check2d(A, "A")
        if A.shape[1] != K:
            raise ValueError("A must be [M,K]")
        a_fmt, lda = BI_A_BF16, A.stride(0)
    else:
        if A.dim() != 2 or A.stride(1) != 1 or A.shape[1] != K // 2:
            raise ValueError("NVFP4 A must be [M,K/2] with unit last stride")
        if tuple(A_scales.shape) != (M, K // 16) or A_scales.stride(1) != 1:
            raise ValueError("A_scales must be [M,K/16]")
        if A_scales.stride(0) * 8 != A.stride(0):
            raise ValueError("A and A_scales row strides must describe the same lda")
        a_fmt, lda = BI_A_NVFP4, A.stride(0) * 2
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=W.device)
    _check2d(Y, "Y")
    st = lib().bi_nvfp4_gemm_ex(_ptr(A), _ptr(A_scales), a_fmt, lda, _ptr(W), _ptr(W_scales),
                                float(alpha), _ptr(Y), Y.stride(0), M, N, K, _stream(stream),
                                _opts(max_workgroups, tile_variant, pipeline_depth, fixed_plan))
    _raise(st, "bi_nvfp4_gemm")
    return Y


def bi_rmsnorm(X, gamma, eps, Y=None, *, stream=None, max_workgroups=0):
    """Y[M,H] = X * rsqrt(mean(X^2) + eps) * gamma, row by row (bf16)."""
    _check2d(X, "X")
    M, H = X.shape
    if gamma.dim() != 1 or gamma.shape[0] != H or not gamma.is_contiguous():
        raise ValueError("gamma must be a dense [H] vector")
    if Y is None:
        Y = torch.empty((M, H), dtype=torch.bfloat16, device=X.device)
    _check2d(Y, "Y")
    st = lib().bi_rmsnorm_ex(_ptr(X), X.stride(0), _ptr(gamma), float(eps), _ptr(Y), Y.stride(0),
                             M, H, _stream(stream), _opts(max_workgroups))
    _raise(st, "bi_rmsnorm")
    return Y


def bi_nvfp4_quant(X, g, Q=None, Q_scales=None, *, stream=None, max_workgroups=0):
    """Row-local NVFP4 quantisation of bf16 X [M,K] with global scale g.

    Returns (Q codes uint8 [M,K/2], Q_scales uint8 [M,K/16]), allocated with
    torch if not given; they are the NVFP4 A operand of bi_nvfp4_gemm.
    """
    _check2d(X, "X")
    M, K = X.shape
    if Q is None:
        Q = torch.empty((M, K // 2), dtype=torch.uint8, device=X.device)
    if Q_scales is None:
        Q_scales = torch.empty((M, K // 16), dtype=torch.uint8, device=X.device)
    if Q.dim() != 2 or Q.stride(1) != 1 or tuple(Q.shape) != (M, K // 2):
        raise ValueError("Q must be [M,K/2] with unit last stride")
    if Q_scales.dim() != 2 or Q_scales.stride(1) != 1 or tuple(Q_scales.shape) != (M, K // 16):
        raise ValueError("Q_scales must be [M,K/16] with unit last stride")
    if Q_scales.stride(0) * 8 != Q.stride(0) and M > 1:
        raise ValueError("Q and Q_scales row strides must describe the same ldq")
    st = lib().bi_nvfp4_quant_ex(_ptr(X), X.stride(0), float(g), _ptr(Q), _ptr(Q_scales),
                                 Q.stride(0) * 2, M, K, _stream(stream), _opts(max_workgroups))
    _raise(st, "bi_nvfp4_quant")
    return Q, Q_scales


def bi_reduce_rmsnorm(partials, gamma, eps, residual=None, R=None, Y=None, *, stream=None,
                      max_workgroups=0):
    """R = residual + partials[0] + ... (fp32, this order, one bf16 rounding);
    Y = RMSNorm(R).  partials: a list of bf16 [M,H] tensors with one common
    row stride.  Returns (R, Y); R may be the residual tensor (in place)."""
    if not partials:
        raise ValueError("at least one partial")
    for t in partials:
        _check2d(t, "partial")
    M, H = partials[0].shape
    ldp = partials[0].stride(0)
    for t in partials:
        if tuple(t.shape) != (M, H) or t.stride(0) != ldp:
            raise ValueError("partials must share shape and row stride")
    if gamma.dim() != 1 or gamma.shape[0] != H or not gamma.is_contiguous():
        raise ValueError("gamma must be a dense [H] vector")
    if residual is not None:
        _check2d(residual, "residual")
        if tuple(residual.shape) != (M, H):
            raise ValueError("residual must be [M,H]")
    if R is None:
        R = torch.empty((M, H), dtype=torch.bfloat16, device=partials[0].device)
    if Y is None:
        Y = torch.empty((M, H), dtype=torch.bfloat16, device=partials[0].device)
    _check2d(R, "R")
    _check2d(Y, "Y")
    arr = (ctypes.c_void_p * len(partials))(*[t.data_ptr() for t in partials])
    st = lib().bi_reduce_rmsnorm_ex(arr, len(partials), ldp, _ptr(residual),
                                    residual.stride(0) if residual is not None else 0, _ptr(gamma),
                                    float(eps), _ptr(R), R.stride(0), _ptr(Y), Y.stride(0), M, H,
                                    _stream(stream), _opts(max_workgroups))
    _raise(st, "bi_reduce_rmsnorm")
    return R, Y


def bi_grouped_gemm(A, W, offsets, Y=None, *, stream=None, max_workgroups=0, tile_variant=0, fixed_plan=False):
    """Mixture-of-experts grouped GEMM: rows offsets[e] .. offsets[e+1]-1 of
    A [T,K] use W[e] [N,K]; offsets is a device int64 tensor [E+1]."""
    _check2d(A, "A")
    if W.dim() != 3 or W.stride(2) != 1:
        raise ValueError("W must be [E,N,K] with unit last stride")
    T, K = A.shape
    E, N, K2 = W.shape
    if K2 != K:
        raise ValueError("A and W disagree on K")
    if offsets.dtype != torch.int64 or offsets.dim() != 1 or offsets.shape[0] != E + 1 or not offsets.is_cuda:
        raise ValueError("offsets must be a device int64 tensor of E+1 entries")
    if Y is None:
        Y = torch.empty((T, N), dtype=torch.bfloat16, device=A.device)
    _check2d(Y, "Y")
    st = lib().bi_grouped_gemm_ex(_ptr(A), A.stride(0), _ptr(W), W.stride(1), W.stride(0), _ptr(Y),
                                  Y.stride(0), _ptr(offsets), E, T, N, K, _stream(stream),
                                  _opts(max_workgroups, tile_variant, 0, fixed_plan))
    _raise(st, "bi_grouped_gemm")
    return Y


def mla_decode_workspace_size(B, H, Lmax, Dqk, Dv) -> int:
    """Bytes of workspace bi_mla_decode uses for this shape (0: none)."""
    n = ctypes.c_int64(0)
    _raise(lib().bi_mla_decode_workspace_size(B, H, Lmax, Dqk, Dv, ctypes.byref(n)), "bi_mla_decode_workspace_size")
    return int(n.value)


def bi_mla_decode(q, kv, lens, scale, Dv, out=None, *, workspace=None, stream=None, max_workgroups=0):
    """Decode attention over a latent KV cache: q bf16 [B,H,Dqk], kv bf16
    [B,Lmax,Dqk], lens a device int32 tensor [B]; returns out bf16 [B,H,Dv]
    = softmax(scale * q . kv^T) . kv[..., :Dv] per request and head.
    workspace: None (one workgroup per request), True (allocate one with
    torch), or a device tensor of at least mla_decode_workspace_size bytes
    (one workgroup per 1024-token chunk when the request and head groups
    leave compute units idle); the bits are the same."""
    for t, name in ((q, "q"), (kv, "kv")):
        if t.dim() != 3 or t.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not t.is_contiguous():
            raise ValueError(f"{name} must be a dense 3-d bf16 tensor")
    B, H, Dqk = q.shape
    B2, Lmax, D2 = kv.shape
    if B2 != B or D2 != Dqk:
        raise ValueError("q and kv disagree on B or Dqk")
    if lens.dtype != torch.int32 or lens.dim() != 1 or lens.shape[0] != B or not lens.is_cuda:
        raise ValueError("lens must be a device int32 tensor of B entries")
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.bfloat16, device=q.device)
    if tuple(out.shape) != (B, H, Dv) or not out.is_contiguous():
        raise ValueError("out must be a dense [B,H,Dv] tensor")
    if workspace is True:
        workspace = torch.empty(max(16, mla_decode_workspace_size(B, H, Lmax, Dqk, Dv)), dtype=torch.uint8,
                                device=q.device)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace),
                                                           workspace.numel() * workspace.element_size())
    st = lib().bi_mla_decode_ex(_ptr(q), _ptr(kv), _ptr(lens), float(scale), _ptr(out), B, H, Lmax, Dqk, Dv,
                                ws_ptr, ws_bytes, _stream(stream), _opts(max_workgroups))
    _raise(st, "bi_mla_decode")
    return out


MLA_SCRATCH_BYTES = 32 << 20  # BI_MLA_SCRATCH_BYTES


def bi_mla_decode_noalloc(q, kv, lens, scale, Dv, out):
    """bi_mla_decode without a workspace and without any allocation: the
    chunked schedule's partials go to the library's per-GPU scratch array.
    `out` (bf16 [B,H,Dv], dense) must be given: nothing is allocated here
    either."""
    for t, name in ((q, "q"), (kv, "kv")):
        if t.dim() != 3 or t.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not t.is_contiguous():
            raise ValueError(f"{name} must be a dense 3-d bf16 tensor")
    B, H, Dqk = q.shape
    B2, Lmax, D2 = kv.shape
    if B2 != B or D2 != Dqk:
        raise ValueError("q and kv disagree on B or Dqk")
    if lens.dtype != torch.int32 or lens.dim() != 1 or lens.shape[0] != B or not lens.is_cuda:
        raise ValueError("lens must be a device int32 tensor of B entries")
    if tuple(out.shape) != (B, H, Dv) or not out.is_contiguous():
        raise ValueError("out must be a dense [B,H,Dv] tensor")
    st = lib().bi_mla_decode_noalloc(_ptr(q), _ptr(kv), _ptr(lens), float(scale), _ptr(out), B, H, Lmax, Dqk,
                                     Dv, _stream(None))
    _raise(st, "bi_mla_decode_noalloc")
    return out


PROBE_WAVES = 8
PROBE_MFMA_FLOPS = 16384  # one v_mfma_f32_16x16x32_bf16


def bi_probe_mfma(iters, grid, out=None, *, stream=None):
    """MFMA-only loop (measurement): returns the device uint64 tensor
    [grid * 8, 3] of (shader-clock cycles, 100 MHz ticks, sink) per wavefront.
    The call performs grid * 8 * iters * 8 * 16384 flops."""
    if out is None:
        out = torch.empty((grid * PROBE_WAVES, 3), dtype=torch.int64, device="cuda")
    _raise(lib().bi_probe_mfma(_ptr(out), int(iters), int(grid), _stream(stream)), "bi_probe_mfma")
    return out


PROBE_LDS_BYTES = 16 * 1024  # LDS bytes one wavefront reads per iteration


def bi_probe_lds(iters, grid, out=None, *, stream=None):
    """LDS read loop (measurement): returns the device uint64 tensor
    [grid * 8, 2] of (shader-clock cycles, sink) per wavefront; each
    wavefront reads iters * 16 KB from LDS."""
    if out is None:
        out = torch.empty((grid * PROBE_WAVES, 2), dtype=torch.int64, device="cuda")
    _raise(lib().bi_probe_lds(_ptr(out), int(iters), int(grid), _stream(stream)), "bi_probe_lds")
    return out


def bi_probe_read(src, grid, sink=None, *, stream=None):
    """Read stream (measurement): reads every byte of the dense device tensor
    src once; returns the uint32 sink tensor [grid * 256]."""
    if not src.is_contiguous():
        raise ValueError("src must be dense")
    if sink is None:
        sink = torch.empty((grid * 256,), dtype=torch.int32, device=src.device)
    _raise(lib().bi_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), int(grid), _stream(stream)),
           "bi_probe_read")
    return sink
