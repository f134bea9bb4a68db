"""fp64 CPU oracle for the batch-invariant GEMM family and RMSNorm.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``invariant_deterministic_bi_amd``) and never
imports it; both sides consume the same stored inputs, produced by the seeded
generators in ``invariant_deterministic_bi_amd.inputs``.

The arithmetic lives in ``oracle.c`` (plain C, fp64, sequential ascending-k
sums); this module only marshals numpy arrays.  Each function returns the
unrounded fp64 result ``y`` and, for the GEMM family, ``s = sum_k |a_k b_k|``
(times |alpha| for NVFP4), the scale of the tolerance
``|y_gpu - y| <= ulp_bf16(y) + 1e-3 * s``.

Parity status: every function is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (integer-exact products, exact rational brute
force, identity/one-hot selection, power-of-two scaling, exhaustive NVFP4
decode tables, RMSNorm closed forms).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.path.join(_HERE, "liboracle.so")
    if not os.path.exists(path):
        _build.build()
    lib = ctypes.CDLL(path)
    lib.oracle_gemm.argtypes = [_p, _i64, _p, _i64, _i64, _i64, _i64, _p, _i64, _p, _p]
    lib.oracle_gemm.restype = None
    lib.oracle_bmm.argtypes = [_p, _i64, _i64, _p, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p]
    lib.oracle_bmm.restype = None
    lib.oracle_nvfp4_gemm.argtypes = [_p, _p, ctypes.c_int, _i64, _p, _p, ctypes.c_float,
                                      _i64, _i64, _i64, _p, _i64, _p, _p]
    lib.oracle_nvfp4_gemm.restype = None
    lib.oracle_rmsnorm.argtypes = [_p, _i64, _p, ctypes.c_float, _i64, _i64, _p, _i64, _p]
    lib.oracle_rmsnorm.restype = None
    lib.oracle_nvfp4_quant.argtypes = [_p, _i64, ctypes.c_float, _i64, _i64, _i64, _p, _p]
    lib.oracle_nvfp4_quant.restype = None
    lib.oracle_reduce_rmsnorm.argtypes = [_p, _i64, _p, _p, ctypes.c_float, _i64, _i64, _p, _p, _p, _p]
    lib.oracle_reduce_rmsnorm.restype = None
    lib.oracle_grouped_gemm.argtypes = [_p, _i64, _p, _i64, _i64, _p, _i64, _i64, _i64, _p, _p]
    lib.oracle_grouped_gemm.restype = None
    lib.oracle_mla_decode.argtypes = [_p, _p, _p, ctypes.c_float, _i64, _i64, _i64, _i64, _i64, _p, _p]
    lib.oracle_mla_decode.restype = None
    for name in ("oracle_e2m1_value", "oracle_e4m3_value", "oracle_bf16_value"):
        getattr(lib, name).argtypes = [ctypes.c_uint32]
        getattr(lib, name).restype = ctypes.c_double
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _u16(a):
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns")
    return a


def _rows(rows):
    if rows is None:
        return None
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return _load().oracle_num_threads()


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits))


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code))


def gemm(A, B, rows=None):
    """y[r, j] = sum_k A[i, k] * B[j, k] with i = rows[r]; A [M,K], B [N,K] bf16 bits.

    Operand orientation y = A . B^T as in the NVFP4 batch-invariance unit test
    of the vLLM PR #39912 summary page (section "key source snippets").
    Returns (y, s) as float64 arrays of shape [len(rows) or M, N].
    """
    A = np.ascontiguousarray(_u16(A))
    B = np.ascontiguousarray(_u16(B))
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    rows = _rows(rows)
    nr = M if rows is None else len(rows)
    if rows is not None:
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < M)
    Y = np.empty((nr, N), np.float64)
    S = np.empty((nr, N), np.float64)
    if nr and N:
        _load().oracle_gemm(_ptr(A), K, _ptr(B), K, M, N, K, _ptr(rows), nr, _ptr(Y), _ptr(S))
    elif N:
        Y[:] = 0
        S[:] = 0
    return Y, S


def bmm(A, B):
    """y[h, i, j] = sum_k A[h, i, k] * B[h, k, j]; A [H,M,K], B [H,K,N] bf16 bits."""
    A = np.ascontiguousarray(_u16(A))
    B = np.ascontiguousarray(_u16(B))
    H, M, K = A.shape
    H2, K2, N = B.shape
    assert H == H2 and K == K2
    Y = np.zeros((H, M, N), np.float64)
    S = np.zeros((H, M, N), np.float64)
    if H and M and N:
        _load().oracle_bmm(_ptr(A), M * K, K, _ptr(B), K * N, N, H, M, N, K, _ptr(Y), _ptr(S))
    return Y, S


def nvfp4_gemm(A, A_scales, W, W_scales, alpha, K, rows=None):
    """y[r, j] = alpha * sum_k a(i, k) * w(j, k) for NVFP4 weights.

    W: uint8 codes [N, K/2] (element 2j in the low nibble of byte j),
    W_scales: uint8 E4M3 [N, K/16].  A is bf16 bits [M, K] when A_scales is
    None, else NVFP4 codes [M, K/2] with scales [M, K/16].  alpha is rounded
    to fp32 first, as the library receives it.
    """
    W = np.ascontiguousarray(np.asarray(W, np.uint8))
    W_scales = np.ascontiguousarray(np.asarray(W_scales, np.uint8))
    N = W.shape[0]
    assert W.shape == (N, K // 2) and W_scales.shape == (N, K // 16)
    if A_scales is None:
        A = np.ascontiguousarray(_u16(A))
        M = A.shape[0]
        assert A.shape == (M, K)
        a_fmt, a_sc = 0, None
    else:
        A = np.ascontiguousarray(np.asarray(A, np.uint8))
        a_sc = np.ascontiguousarray(np.asarray(A_scales, np.uint8))
        M = A.shape[0]
        assert A.shape == (M, K // 2) and a_sc.shape == (M, K // 16)
        a_fmt = 1
    rows = _rows(rows)
    nr = M if rows is None else len(rows)
    Y = np.zeros((nr, N), np.float64)
    S = np.zeros((nr, N), np.float64)
    if nr and N:
        _load().oracle_nvfp4_gemm(_ptr(A), _ptr(a_sc), a_fmt, K, _ptr(W), _ptr(W_scales),
                                  float(np.float32(alpha)), M, N, K, _ptr(rows), nr,
                                  _ptr(Y), _ptr(S))
    return Y, S


def rmsnorm(X, gamma, eps, rows=None):
    """y[r, h] = x[i, h] * gamma[h] / sqrt(mean_h' x[i, h']^2 + eps), fp64.

    X [M,H] and gamma [H] are bf16 bits; eps is rounded to fp32 first, as the
    library receives it.
    """
    X = np.ascontiguousarray(_u16(X))
    gamma = np.ascontiguousarray(_u16(gamma))
    M, H = X.shape
    assert gamma.shape == (H,)
    rows = _rows(rows)
    nr = M if rows is None else len(rows)
    Y = np.zeros((nr, H), np.float64)
    if nr and H:
        _load().oracle_rmsnorm(_ptr(X), H, _ptr(gamma), float(np.float32(eps)), M, H,
                               _ptr(rows), nr, _ptr(Y))
    return Y


def nvfp4_quant(X, global_scale):
    """Row-local NVFP4 quantisation of bf16 activations X [M, K] (K % 16 == 0).

    The quantiser named in the unit test of the vLLM PR #39912 summary page
    (section "key source snippets"), in the fp32 reading spelled out in
    oracle.c: per 16-element block, scale = nearest E4M3 to
    min(fp32(fp32(amax * g) / 6), 448); codes = nearest E2M1 to
    fp32(|x| * fp32(g / scale)), ties to even codes.  global_scale is rounded
    to fp32 first, as the library receives it.  Returns (codes uint8
    [M, K/2], scales uint8 [M, K/16]).
    """
    X = np.ascontiguousarray(_u16(X))
    M, K = X.shape
    assert K % 16 == 0
    Q = np.zeros((M, K // 2), np.uint8)
    S = np.zeros((M, K // 16), np.uint8)
    if M and K:
        _load().oracle_nvfp4_quant(_ptr(X), K, float(np.float32(global_scale)), M, K, K,
                                   _ptr(Q), _ptr(S))
    return Q, S


def reduce_rmsnorm(partials, gamma, eps, residual=None):
    """Fixed-order reduction of partial outputs followed by RMSNorm, fp64.

    partials: bf16 bits [P, M, H] (the per-rank partial outputs of a
    row-parallel layer); residual: bf16 bits [M, H] or None; gamma [H].
    R = residual + sum_p partials[p]; Y = R * gamma / sqrt(mean_h R^2 + eps)
    (the all-reduce + RMSNorm pair of the vLLM PR #51292 page, section
    "Purpose").  eps is rounded to fp32 first.  Returns (R, SR, Y, SY):
    SR = sum of |terms| of each R element, SY = |gamma| * SR / rms, the
    scales of the tolerances.
    """
    P = np.ascontiguousarray(_u16(partials))
    gamma = np.ascontiguousarray(_u16(gamma))
    n, M, H = P.shape
    assert gamma.shape == (H,)
    res = None
    if residual is not None:
        res = np.ascontiguousarray(_u16(residual))
        assert res.shape == (M, H)
    R = np.zeros((M, H), np.float64)
    SR = np.zeros((M, H), np.float64)
    Y = np.zeros((M, H), np.float64)
    SY = np.zeros((M, H), np.float64)
    if M and H:
        _load().oracle_reduce_rmsnorm(_ptr(P), n, _ptr(res), _ptr(gamma), float(np.float32(eps)),
                                      M, H, _ptr(R), _ptr(SR), _ptr(Y), _ptr(SY))
    return R, SR, Y, SY


def grouped_gemm(A, W, offsets):
    """Mixture-of-experts grouped GEMM: rows offsets[e] .. offsets[e+1]-1 of
    A [T, K] (bf16 bits) use expert e's weight W[e] [N, K];
    y[t, j] = sum_k A[t, k] * W[e(t), j, k].  Returns (y, s) [T, N] fp64."""
    A = np.ascontiguousarray(_u16(A))
    W = np.ascontiguousarray(_u16(W))
    off = np.ascontiguousarray(np.asarray(offsets, np.int64))
    T, K = A.shape
    E, N, K2 = W.shape
    assert K == K2 and off.shape == (E + 1,) and off[0] == 0 and off[-1] == T
    assert np.all(np.diff(off) >= 0)
    Y = np.zeros((T, N), np.float64)
    S = np.zeros((T, N), np.float64)
    if T and N:
        _load().oracle_grouped_gemm(_ptr(A), K, _ptr(W), K, N * K, _ptr(off), E, N, K, _ptr(Y), _ptr(S))
    return Y, S


def mla_decode(q, kv, lens, scale, Dv):
    """Decode attention over a latent KV cache, fp64 plain definition:
    s_t = scale * q . kv_t (all Dqk components), p = softmax(s) over the
    request's L_b tokens, o = sum_t p_t * kv_t[:Dv].  q bf16 [B, H, Dqk],
    kv bf16 [B, Lmax, Dqk], lens [B].  scale is rounded to fp32 first.
    Returns (o, s) [B, H, Dv], s = sum_t p_t |v_t| (tolerance scale)."""
    q = np.ascontiguousarray(_u16(q))
    kv = np.ascontiguousarray(_u16(kv))
    lens = np.ascontiguousarray(np.asarray(lens, np.int64))
    B, H, Dqk = q.shape
    B2, Lmax, D2 = kv.shape
    assert B == B2 and Dqk == D2 and lens.shape == (B,) and 0 < Dv <= Dqk
    assert np.all((lens >= 0) & (lens <= Lmax))
    O = np.zeros((B, H, Dv), np.float64)
    S = np.zeros((B, H, Dv), np.float64)
    if B and H:
        _load().oracle_mla_decode(_ptr(q), _ptr(kv), _ptr(lens), float(np.float32(scale)), B, H, Lmax,
                                  Dqk, Dv, _ptr(O), _ptr(S))
    return O, S
