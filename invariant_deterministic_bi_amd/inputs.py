"""Seeded synthetic inputs for the batch-invariant GEMM family and RMSNorm.

This module only makes inputs: bf16 bit patterns drawn from seeded
distributions, and NVFP4 weight/activation encodings produced by a host
quantiser.  It holds none of the arithmetic of the operations themselves, and
it imports neither the HIP binding nor the oracle, so both can consume what it
produces.

Conventions:
  * every array is returned as raw bit patterns: bf16 as ``uint16``, NVFP4
    codes and E4M3 scales as ``uint8``;
  * randomness is numpy's PCG64 seeded from ``(seed, tag...)`` through a
    ``SeedSequence``, so each tensor of a workload has its own stream;
  * the default seed is 12345, the default of the test seed variable in the
    vLLM PR #39912 unit test (summary page, section "key source snippets");
  * real values are drawn in fp64, rounded to fp32 (round-to-nearest-even),
    then to bf16 (round-to-nearest-even on the bit pattern).

NVFP4 layout (the pages give only ``k = 2 * packed_k`` for the packed
codes): element 2j of a row sits in the low nibble of byte j, element 2j+1 in
the high nibble; one E4M3 scale byte covers 16 consecutive elements of a row;
codes are ``[rows, K/2]`` and scales ``[rows, K/16]``, both row-major.
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 12345


def rng(seed: int = BASE_SEED, *tag: int) -> np.random.Generator:
    """A PCG64 generator for the stream (seed, *tag)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, tag)])))


def to_bf16_bits(x) -> np.ndarray:
    """Round real values to bf16: fp64 -> fp32 (RNE) -> bf16 (RNE), as uint16 bits."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def randn_bf16(shape, std: float = 1.0, seed: int = BASE_SEED, tag=(0,)) -> np.ndarray:
    """N(0, std^2) samples rounded to bf16."""
    return to_bf16_bits(rng(seed, *tag).standard_normal(shape) * std)


def uniform_bf16(shape, lo: float, hi: float, seed: int = BASE_SEED, tag=(0,)) -> np.ndarray:
    """U(lo, hi) samples rounded to bf16."""
    return to_bf16_bits(rng(seed, *tag).uniform(lo, hi, size=shape))


def randint_bf16(shape, lo: int, hi: int, seed: int = BASE_SEED, tag=(0,)) -> np.ndarray:
    """Integers drawn uniformly from [lo, hi], stored as bf16 (exact for |v| <= 256)."""
    assert -256 <= lo <= hi <= 256
    return to_bf16_bits(rng(seed, *tag).integers(lo, hi + 1, size=shape).astype(np.float64))


# --------------------------------------------------------------------------
# NVFP4 host quantiser (input preparation).
#
# The pages use a per-tensor global scale and a quantiser returning packed
# FP4 codes plus per-16 block scales, without defining either.  Reading used
# here: g = 448 * 6 / amax|X| (maps the tensor's largest magnitude onto the
# largest product of an E4M3 scale and an E2M1 value); per 16-element block,
# scale s = E4M3_RNE(min(amax_blk * g / 6, 448)); element code
# q = E2M1_RNE(|x| * (g / s)) with the sign of x, saturating at 6, ties to
# even, q = 0 when s = 0.
# The GEMM consumes only the stored codes, so this choice cannot move parity.
# --------------------------------------------------------------------------

def _e2m1_magnitudes() -> np.ndarray:
    """Magnitudes of FP4 E2M1 codes 0..7 from the bit layout (exp bias 1)."""
    out = []
    for c in range(8):
        e, m = c >> 1, c & 1
        out.append(0.5 * m if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1))
    return np.array(out)


def _e4m3_magnitudes() -> np.ndarray:
    """Magnitudes of FP8 E4M3 codes 0..126 (the finite non-negative ones)."""
    out = []
    for c in range(127):
        e, m = c >> 3, c & 7
        out.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(out)


_E2M1 = _e2m1_magnitudes()
_E4M3 = _e4m3_magnitudes()


def _round_to_table(v: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the nearest table entry to each v >= 0 (table ascending, index
    = code), ties to the even code, values beyond the last entry saturate."""
    v = np.minimum(v, table[-1])
    hi = np.clip(np.searchsorted(table, v, side="left"), 0, len(table) - 1)
    lo = np.clip(hi - 1, 0, len(table) - 1)
    dlo = v - table[lo]
    dhi = table[hi] - v
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo).astype(np.int64)


def nvfp4_global_scale(x) -> np.float32:
    """Per-tensor global scale 448*6/amax|x| as fp32 (1.0 for an all-zero tensor)."""
    amax = float(np.max(np.abs(np.asarray(x, np.float64)))) if np.size(x) else 0.0
    return np.float32(1.0) if amax == 0.0 else np.float32(448.0 * 6.0 / amax)


def _e2m1_rne_code(t: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code (0..7) nearest to t >= 0, ties to the even code,
    saturating at 6.  The decision points are the midpoints between adjacent
    magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; at a midpoint the even code wins,
    hence '>' where the lower neighbour is even and '>=' where the upper is."""
    mids = ((0.25, False), (0.75, True), (1.25, False), (1.75, True),
            (2.5, False), (3.5, True), (5.0, False))
    code = np.zeros(t.shape, np.uint8)
    for m, upper_even in mids:
        code += (t >= m) if upper_even else (t > m)
    return code


def nvfp4_quantize(x, global_scale) -> tuple[np.ndarray, np.ndarray]:
    """Quantise real values x [R, K] (K % 16 == 0) with a given global scale.

    Returns (codes uint8 [R, K/2], scales uint8 [R, K/16]).  Each row depends
    only on itself and the global scale, so quantising a row alone with the
    same global scale gives the same bytes as quantising it inside a batch.
    Large inputs are processed in row blocks to bound host memory.
    """
    x = np.asarray(x)
    R, K = x.shape
    assert K % 16 == 0
    g = float(np.float32(global_scale))
    codes = np.empty((R, K // 2), np.uint8)
    scales = np.empty((R, K // 16), np.uint8)
    step = max(1, (1 << 22) // K)
    for r0 in range(0, R, step):
        blk = np.asarray(x[r0:r0 + step], np.float64).reshape(-1, K // 16, 16)
        amax = np.max(np.abs(blk), axis=2)
        s_code = _round_to_table(np.minimum(amax * g / 6.0, 448.0), _E4M3)
        s_val = _E4M3[s_code]
        inv = np.where(s_val > 0, g / np.where(s_val > 0, s_val, 1.0), 0.0)
        q = _e2m1_rne_code(np.abs(blk) * inv[..., None])
        q = np.where(np.signbit(blk) & (q != 0), q | np.uint8(8), q).reshape(-1, K)
        codes[r0:r0 + step] = q[:, 0::2] | (q[:, 1::2] << np.uint8(4))
        scales[r0:r0 + step] = s_code.astype(np.uint8)
    return codes, scales


def random_nvfp4_pow2(shape, seed: int = BASE_SEED, tag=(0,), exp_range=(-3, 3)):
    """Random NVFP4 codes with E4M3 scales restricted to powers of two.

    Every element is then k/2 * 2^e for small integers, so products with
    small-integer bf16 activations and their sums are exact in fp32.
    Returns (codes [R, K/2], scales [R, K/16]).
    """
    R, K = shape
    g = rng(seed, *tag)
    q = g.integers(0, 16, size=(R, K))
    e = g.integers(exp_range[0], exp_range[1] + 1, size=(R, K // 16))
    s_code = ((e + 7) << 3).astype(np.uint8)  # exponent field e+7, mantissa 0
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return codes, s_code
