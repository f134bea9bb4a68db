"""Shared test helpers: bf16 decoding of results, the tolerance, comparisons.

The tolerance for the GEMM family is |y - y_ref| <= ulp_bf16(y_ref) +
1e-3 * sum_k |a_k b_k|; for RMSNorm the same form with one product term,
|y - y_ref| <= ulp_bf16(y_ref) + 1e-3 * |y_ref|.
"""
import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits).view(np.uint16) if np.asarray(bits).dtype == np.int16 else np.asarray(bits, np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def ulp_bf16(y) -> np.ndarray:
    """Spacing of bf16 at |y|: 2^(max(floor(log2|y|), -126) - 7); 2^-133 at 0."""
    a = np.abs(np.asarray(y, np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, -126.0), -126.0)
    return np.exp2(e - 7.0)


def tol_excess(y_gpu_bits, y_ref, s, rel=1e-3):
    """max over elements of |y - y_ref| - (ulp(y_ref) + rel*s); <= 0 passes."""
    y = bf16_to_f64(y_gpu_bits)
    err = np.abs(y - y_ref)
    bound = ulp_bf16(y_ref) + rel * np.asarray(s, np.float64)
    if err.size == 0:
        return -1.0
    return float(np.max(err - bound))


def assert_within_tol(y_gpu_bits, y_ref, s, what="", extra=None):
    """|y - y_ref| <= ulp_bf16(y_ref) + 1e-3 * s (+ extra, an error term a
    reading adds, e.g. an intermediate bf16 rounding the method performs)."""
    y = bf16_to_f64(y_gpu_bits)
    assert y.shape == np.shape(y_ref), (what, y.shape, np.shape(y_ref))
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - y_ref)
    bound = ulp_bf16(y_ref) + 1e-3 * np.asarray(s, np.float64)
    if extra is not None:
        bound = bound + extra
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at {tuple(idx)}: "
            f"gpu={y[tuple(idx)]!r} ref={y_ref[tuple(idx)]!r} bound={bound[tuple(idx)]!r}")


def rne_bf16_of_exact(y_exact) -> np.ndarray:
    """bf16 bits of exactly representable-in-fp32 values, rounded to nearest even."""
    f = np.asarray(y_exact, np.float64).astype(np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(y_exact, np.float64)), "not exact in fp32"
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def reduce_rms_y_extra(R_ref, gamma_bits, eps):
    """Extra tolerance of Y = RMSNorm(R) when R is materialised in bf16 first
    (the reduced tensor, as an all-reduce returns it): rounding R costs at most
    half a bf16 ulp of R, which reaches y scaled by |gamma| / rms(R)."""
    R = np.asarray(R_ref, np.float64)
    rms = np.sqrt(np.mean(R * R, axis=-1, keepdims=True) + float(np.float32(eps)))
    g = np.abs(bf16_to_f64(gamma_bits))
    return 0.5 * ulp_bf16(R) * g / rms


def mla_rel_bound(q_bits, kv_bits, lens, scale):
    """First-order rounding bound of the fp32 decode attention, as a multiple
    c[b,h] of S = sum_t p_t |v_t| / sum_t p_t, from the inputs alone (u =
    2^-24).  A weight's relative error is at most that of its score
    (Dqk*u*A, A = |scale| * max_t sum_d |q_d kv_td|), of the exp2 argument
    (u*|s - m| <= 2u*A) and of exp2 itself (2u); it moves the output by at
    most twice that times S.  The value chains (L/4 + 3 steps) and the weight
    sum (L + 8 steps) add (5L/4 + 11)*u, the division u.  The matrix-core
    path adds the split of each weight into two bf16 parts (2^-18 relative,
    twice) and one rescaling per 32-token block and per merged wave
    ((L/32 + 8)*u).  Returns max(1e-3, 1.01 * c), broadcast over Dv."""
    qf = np.abs(bf16_to_f64(q_bits))
    kf = np.abs(bf16_to_f64(kv_bits))
    Bn, H, Dqk = qf.shape
    u = 2.0 ** -24
    c = np.zeros((Bn, H, 1))
    for b in range(Bn):
        L = int(lens[b])
        if L == 0:
            continue
        A = abs(float(scale)) * np.max(qf[b] @ kf[b, :L].T, axis=1)
        c[b, :, 0] = (2 * (Dqk * u * A + 2 * u * A + 2 * u + 2.0 ** -18) + (1.25 * L + 11) * u + u
                      + (L / 32 + 8) * u)
    return np.maximum(1e-3, 1.01 * c)
