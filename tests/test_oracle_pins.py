"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test ties one oracle function to something independent: hand-worked
examples (tests/golden/worked_examples.txt), a published format table
(tests/golden/e2m1_ocp_mx.txt), a library routine (torch's float8/bfloat16
conversions, numpy integer matmul), exact rational brute force
(fractions.Fraction), closed forms and invariants.  They are chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a misplaced scale or nibble) fails at least one.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_bi_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _parse_matrix(txt):
    return [[float(v) for v in row.split(",")] for row in txt.split(";")]


def _worked():
    out = {}
    with open(os.path.join(GOLDEN, "worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, rest = [p.strip() for p in line.split(":", 1)]
            lhs, rhs = [p.strip() for p in rest.split("=>")]
            args = dict(tok.split("=", 1) for tok in lhs.split())
            out[name] = (args, rhs)
    return out


WORKED = _worked()


def bits(values):
    return inputs.to_bf16_bits(np.asarray(values, np.float64))


def torch_bf16_value(b):
    t = torch.from_numpy(np.asarray(b, np.uint16).astype(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------- decoders

def test_bf16_decode_matches_torch_exhaustive():
    allbits = np.arange(65536, dtype=np.uint32)
    ours = np.array([oracle.bf16_value(int(b)) for b in allbits[::97]])
    ref = torch_bf16_value(allbits[::97].astype(np.uint16))
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.all(both_nan | (ours == ref))
    # a few hand-checked patterns (IEEE binary32 upper halves)
    assert oracle.bf16_value(0x3F80) == 1.0
    assert oracle.bf16_value(0xC000) == -2.0
    assert oracle.bf16_value(0x4049) == 3.140625
    assert oracle.bf16_value(0x0001) == 2.0 ** -133
    assert oracle.bf16_value(0x7F7F) == (2 - 2 ** -7) * 2.0 ** 127


def test_e2m1_decode_matches_ocp_table():
    table = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                table[int(c, 16)] = float(v)
    assert len(table) == 16
    for c, v in table.items():
        got = oracle.e2m1_value(c)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (c, got, v)


def test_e4m3_decode_matches_torch_exhaustive():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0xB8) == -1.0


def test_nvfp4_products_exact_in_bf16():
    """Every e2m1 x e4m3 product (4096 of them) is a bf16 value: <= 6
    significant bits, magnitudes in [2^-10, 2688]."""
    for q in range(16):
        for s in range(256):
            if s in (0x7F, 0xFF):
                continue
            v = oracle.e2m1_value(q) * oracle.e4m3_value(s)
            b = inputs.to_bf16_bits(np.array([v]))
            assert torch_bf16_value(b)[0] == v, (q, s, v)
            if v != 0:
                assert 2.0 ** -10 <= abs(v) <= 2688.0


# ---------------------------------------------------------------- GEMM

def test_gemm_worked_examples():
    for name in ("gemm_orient", "gemm_small"):
        args, rhs = WORKED[name]
        A = bits(_parse_matrix(args["A"]))
        B = bits(_parse_matrix(args["B"]))
        y, s = oracle.gemm(A, B)
        assert np.array_equal(y, np.array(_parse_matrix(rhs))), name


@pytest.mark.parametrize("M,N,K", [(7, 33, 544), (1, 256, 512), (5, 3, 12288)])
def test_gemm_integer_exact(M, N, K):
    A = inputs.randint_bf16((M, K), -3, 3, tag=(1, M, N, K))
    B = inputs.randint_bf16((N, K), -3, 3, tag=(2, M, N, K))
    Ai = torch_bf16_value(A).astype(np.int64)
    Bi = torch_bf16_value(B).astype(np.int64)
    y, s = oracle.gemm(A, B)
    assert np.array_equal(y, (Ai @ Bi.T).astype(np.float64))
    assert np.array_equal(s, (np.abs(Ai) @ np.abs(Bi).T).astype(np.float64))


def test_gemm_bruteforce_fraction():
    M, N, K = 3, 4, 37
    A = inputs.randn_bf16((M, K), tag=(3,))
    B = inputs.randn_bf16((N, K), tag=(4,))
    av, bv = torch_bf16_value(A), torch_bf16_value(B)
    y, s = oracle.gemm(A, B)
    u = 2.0 ** -53
    gamma = K * u / (1 - K * u)
    for i in range(M):
        for j in range(N):
            exact = sum(Fraction(av[i, k]) * Fraction(bv[j, k]) for k in range(K))
            sabs = sum(abs(Fraction(av[i, k]) * Fraction(bv[j, k])) for k in range(K))
            assert abs(Fraction(y[i, j]) - exact) <= Fraction(gamma) * sabs
            assert abs(Fraction(s[i, j]) - sabs) <= Fraction(gamma) * sabs
            fs = math.fsum(float(av[i, k]) * float(bv[j, k]) for k in range(K))
            assert abs(y[i, j] - fs) <= gamma * float(sabs)


def test_gemm_identity_and_one_hot():
    K = 64
    A = inputs.randn_bf16((9, K), tag=(5,))
    I = bits(np.eye(K))
    y, _ = oracle.gemm(A, I)
    assert np.array_equal(y, torch_bf16_value(A))
    B = inputs.randn_bf16((17, K), tag=(6,))
    for k in (0, 13, K - 1):
        e = np.zeros((1, K))
        e[0, k] = 1.0
        y, _ = oracle.gemm(bits(e), B)
        assert np.array_equal(y[0], torch_bf16_value(B)[:, k])


def test_gemm_rows_and_permutation():
    A = inputs.randn_bf16((23, 96), tag=(7,))
    B = inputs.randn_bf16((11, 96), tag=(8,))
    y, s = oracle.gemm(A, B)
    perm = inputs.rng(12345, 9).permutation(23)
    yp, sp = oracle.gemm(A[perm], B)
    assert np.array_equal(yp, y[perm]) and np.array_equal(sp, s[perm])
    rows = [22, 0, 5, 5]
    yr, sr = oracle.gemm(A, B, rows=rows)
    assert np.array_equal(yr, y[rows]) and np.array_equal(sr, s[rows])


def test_gemm_power_of_two_scaling():
    A = inputs.randn_bf16((4, 128), tag=(10,))
    B = inputs.randn_bf16((6, 128), tag=(11,))
    y, _ = oracle.gemm(A, B)
    y8, _ = oracle.gemm(bits(torch_bf16_value(A) * 8), B)
    assert np.array_equal(y8, 8 * y)


# ---------------------------------------------------------------- BMM

def test_bmm_worked_example():
    args, rhs = WORKED["bmm_two_heads"]
    A = bits([_parse_matrix(h) for h in args["A"].split("|")])
    B = bits([_parse_matrix(h) for h in args["B"].split("|")])
    y, _ = oracle.bmm(A, B)
    want = np.array([_parse_matrix(h) for h in rhs.split("|")])
    assert np.array_equal(y, want)


def test_bmm_integer_exact():
    H, M, K, N = 5, 7, 128, 40
    A = inputs.randint_bf16((H, M, K), -3, 3, tag=(12,))
    B = inputs.randint_bf16((H, K, N), -3, 3, tag=(13,))
    Ai, Bi = torch_bf16_value(A).astype(np.int64), torch_bf16_value(B).astype(np.int64)
    y, s = oracle.bmm(A, B)
    assert np.array_equal(y, np.matmul(Ai, Bi).astype(np.float64))
    assert np.array_equal(s, np.matmul(np.abs(Ai), np.abs(Bi)).astype(np.float64))


# ---------------------------------------------------------------- NVFP4

def _decode_nvfp4_independent(codes, scales, K):
    """Decode with the OCP golden table and torch's float8_e4m3fn."""
    table = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                table[int(c, 16)] = float(v)
    lut = np.array([table[c] for c in range(16)])
    R = codes.shape[0]
    q = np.empty((R, K), np.int64)
    q[:, 0::2] = codes & 15
    q[:, 1::2] = codes >> 4
    sv = torch.from_numpy(scales.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return lut[q] * np.repeat(sv, 16, axis=1)


def test_nvfp4_nibble_order_worked_example():
    K = 16
    W = np.zeros((1, K // 2), np.uint8)
    W[0, 0] = 0x21
    Ws = np.full((1, 1), 0x40, np.uint8)
    for k, want in ((0, 1.0), (1, 2.0), (2, 0.0)):
        e = np.zeros((1, K))
        e[0, k] = 1.0
        y, s = oracle.nvfp4_gemm(bits(e), None, W, Ws, 1.0, K)
        assert y[0, 0] == want and s[0, 0] == abs(want)


@pytest.mark.parametrize("a_fmt", ["bf16", "nvfp4"])
def test_nvfp4_exact_pow2(a_fmt):
    M, N, K = 6, 21, 256
    W, Ws = inputs.random_nvfp4_pow2((N, K), tag=(14,))
    if a_fmt == "bf16":
        A = inputs.randint_bf16((M, K), -3, 3, tag=(15,))
        As = None
        a_val = torch_bf16_value(A)
    else:
        A, As = inputs.random_nvfp4_pow2((M, K), tag=(16,))
        a_val = _decode_nvfp4_independent(A, As, K)
    w_val = _decode_nvfp4_independent(W, Ws, K)
    want = a_val @ w_val.T  # exact: dyadic values with few bits
    for alpha in (1.0, 0.25, -2.0):
        y, s = oracle.nvfp4_gemm(A, As, W, Ws, alpha, K)
        assert np.array_equal(y, alpha * want)
        assert np.array_equal(s, abs(alpha) * (np.abs(a_val) @ np.abs(w_val).T))


def test_nvfp4_gaussian_vs_dequantised_gemm_bound():
    """Quantised weights: the oracle equals the exact dot of decoded values."""
    M, N, K = 2, 5, 64
    x = inputs.rng(12345, 17).standard_normal((N, K)) * 0.02
    g = inputs.nvfp4_global_scale(x)
    W, Ws = inputs.nvfp4_quantize(x, g)
    A = inputs.randn_bf16((M, K), tag=(18,))
    w_val = _decode_nvfp4_independent(W, Ws, K)
    a_val = torch_bf16_value(A)
    alpha = float(np.float32(1.0 / g))
    y, s = oracle.nvfp4_gemm(A, None, W, Ws, alpha, K)
    for i in range(M):
        for j in range(N):
            exact = alpha * sum(Fraction(a_val[i, k]) * Fraction(w_val[j, k]) for k in range(K))
            assert abs(Fraction(y[i, j]) - exact) <= Fraction(1e-13) * (1 + abs(exact))


# ---------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("name", ["rmsnorm_34", "rmsnorm_ones", "rmsnorm_single"])
def test_rmsnorm_worked_examples(name):
    args, rhs = WORKED[name]
    x = bits([[float(v) for v in args["x"].split(",")]])
    gam = bits([float(v) for v in args["gamma"].split(",")])
    y = oracle.rmsnorm(x, gam, float(args["eps"]))
    want = np.array([float(v) for v in rhs.split(",")])
    assert np.allclose(y[0], want, rtol=1e-15, atol=0), (y, want)


def test_rmsnorm_closed_forms():
    H = 512
    gam = inputs.uniform_bf16((H,), 0.5, 1.5, tag=(19,))
    gv = torch_bf16_value(gam)
    eps = 1e-6
    e32 = float(np.float32(eps))
    rows = np.stack([
        np.zeros(H),                                   # zero row -> 0
        np.full(H, 0.75),                              # constant row
        np.where(np.arange(H) % 3 == 0, -4.0, 4.0),    # +-2^p row
    ])
    y = oracle.rmsnorm(bits(rows), gam, eps)
    assert np.array_equal(y[0], np.zeros(H))
    assert np.allclose(y[1], gv * 0.75 / math.sqrt(0.75 ** 2 + e32), rtol=1e-15)
    assert np.allclose(y[2], np.sign(rows[2]) * gv * 4 / math.sqrt(16 + e32), rtol=1e-15)


def test_rmsnorm_scale_invariance_and_rows():
    X = inputs.randn_bf16((9, 256), tag=(20,))
    gam = inputs.uniform_bf16((256,), 0.5, 1.5, tag=(21,))
    y = oracle.rmsnorm(X, gam, 0.0)
    y4 = oracle.rmsnorm(bits(torch_bf16_value(X) * 4), gam, 0.0)
    assert np.array_equal(y, y4)
    yr = oracle.rmsnorm(X, gam, 1e-6, rows=[8, 1])
    yf = oracle.rmsnorm(X, gam, 1e-6)
    assert np.array_equal(yr, yf[[8, 1]])


# ---------------------------------------------------------------- generators

def test_bf16_rounding_matches_torch():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 257.0, 259.0, -3.3, 1e-40, 6.1e4])
    ours = inputs.to_bf16_bits(vals)
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    x = inputs.rng(12345, 22).standard_normal(10000)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(inputs.to_bf16_bits(x), ref)


def test_generators_deterministic():
    a = inputs.randn_bf16((4, 8), tag=(1, 2))
    b = inputs.randn_bf16((4, 8), tag=(1, 2))
    c = inputs.randn_bf16((4, 8), tag=(1, 3))
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_quantiser_row_local_and_error_bound():
    x = inputs.rng(12345, 23).standard_normal((8, 64)) * 0.02
    g = inputs.nvfp4_global_scale(x)
    W, Ws = inputs.nvfp4_quantize(x, g)
    for i in range(8):
        Wi, Wsi = inputs.nvfp4_quantize(x[i:i + 1], g)
        assert np.array_equal(Wi[0], W[i]) and np.array_equal(Wsi[0], Ws[i])
    dec = _decode_nvfp4_independent(W, Ws, 64) / float(g)
    # each element within half an e2m1 step of its block scale (plus scale rounding)
    blk_amax = np.repeat(np.abs(x).reshape(8, 4, 16).max(axis=2), 16, axis=1)
    assert np.all(np.abs(dec - x) <= blk_amax * 0.25 + 1e-12)


# ---------------------------------------------------------------- NVFP4 quantiser (activations)
#
# oracle.nvfp4_quant is the row-local quantiser of the W4A4 path (the
# scaled_fp4_quant step of the vLLM PR #39912 unit test, summary page,
# section "key source snippets"), in the fp32 reading stated in oracle.c.
# Pins: hand-worked examples, torch's own float8_e4m3fn rounding for the
# scale, exact rational nearest-value search for both codes away from
# decision midpoints, decode-then-requantise round trips, power-of-two
# scaling and row independence.

def _quant_examples():
    out = {}
    with open(os.path.join(GOLDEN, "nvfp4_quant_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, rest = [p.strip() for p in line.split(":", 1)]
            lhs, rhs = [p.strip() for p in rest.split("=>")]
            args = dict(tok.split("=", 1) for tok in lhs.split())
            want = dict(tok.split("=", 1) for tok in rhs.split())
            x = [float(v) for v in args["x"].split(",")]
            codes = np.array([int(b, 16) for b in want["codes"].split(",")], np.uint8)
            scales = np.array([int(b, 16) for b in want["scales"].split(",")], np.uint8)
            out[name] = (float(args["g"]), x, codes, scales)
    return out


QUANT_EXAMPLES = _quant_examples()


@pytest.mark.parametrize("name", sorted(QUANT_EXAMPLES))
def test_nvfp4_quant_worked_examples(name):
    g, x, codes, scales = QUANT_EXAMPLES[name]
    xb = bits([x])
    assert np.array_equal(inputs.bf16_bits_to_f32(xb)[0], np.float32(x)), "example not exact in bf16"
    q, s = oracle.nvfp4_quant(xb, g)
    assert q[0].tolist() == codes.tolist(), (name, [hex(v) for v in q[0]])
    assert s[0].tolist() == scales.tolist(), (name, [hex(v) for v in s[0]])


def _e4m3_table():
    return torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _e2m1_table():
    return [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _nearest_exact(v, table):
    """(code, distance to the nearest decision midpoint) for a Fraction v >= 0,
    by exact scan: nearest table entry, ties to the even code."""
    best, bd = 0, abs(Fraction(table[0]) - v)
    for c in range(1, len(table)):
        d = abs(Fraction(table[c]) - v)
        if d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    mids = [(Fraction(table[c]) + Fraction(table[c + 1])) / 2 for c in range(len(table) - 1)]
    return best, min(abs(v - m) for m in mids)


def test_nvfp4_quant_scale_matches_torch_float8_rounding():
    """The scale byte equals torch's own fp32 -> float8_e4m3fn conversion
    (round to nearest even) of min(fp32(fp32(amax*g)/6), 448)."""
    x = inputs.randn_bf16((64, 256), 1.0, tag=(31,))
    xf = inputs.bf16_bits_to_f32(x)
    for g in (np.float32(448 * 6 / np.abs(xf).max()), np.float32(1.0), np.float32(3.0e-3),
              np.float32(0.37)):
        q, s = oracle.nvfp4_quant(x, g)
        amax = np.abs(xf).reshape(64, 16, 16).max(axis=2).astype(np.float32)
        v = np.minimum((amax * g).astype(np.float32) / np.float32(6.0), np.float32(448.0)).astype(np.float32)
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(s, ref), float(g)


def test_nvfp4_quant_exact_rational_away_from_midpoints():
    """Against exact arithmetic: the scale code is the E4M3 code nearest to
    amax*g/6 and each element code the E2M1 code nearest to |x|*g/s, wherever
    the exact value is not within 2^-20 (relative) of a decision midpoint, where
    the fp32 roundings of the reading may legitimately move it."""
    e4 = _e4m3_table()
    e2 = _e2m1_table()
    x = inputs.randn_bf16((12, 64), 1.0, tag=(32,))
    xf = inputs.bf16_bits_to_f32(x).astype(np.float64)
    checked = skipped = 0
    for g in (np.float32(448 * 6 / np.abs(xf).max()), np.float32(0.8), np.float32(2.0e-3)):
        q, s = oracle.nvfp4_quant(x, g)
        G = Fraction(float(g))
        for i in range(x.shape[0]):
            for b in range(x.shape[1] // 16):
                blk = [Fraction(float(v)) for v in xf[i, 16 * b:16 * b + 16]]
                amax = max(abs(v) for v in blk)
                vstar = min(amax * G / 6, Fraction(448))
                code, dist = _nearest_exact(vstar, e4)
                if vstar > 0 and dist <= vstar * Fraction(1, 1 << 20):
                    skipped += 1
                    continue
                assert s[i, b] == code, (float(g), i, b, float(vstar), s[i, b], code)
                checked += 1
                sv = Fraction(float(e4[code]))
                for j, xv in enumerate(blk):
                    k = 16 * b + j
                    got = (q[i, k // 2] >> (4 * (k % 2))) & 15
                    if sv == 0:
                        assert got == 0
                        continue
                    w = abs(xv) * G / sv
                    c, d = _nearest_exact(w, e2)
                    if w > 0 and d <= w * Fraction(1, 1 << 20):
                        skipped += 1
                        continue
                    want = c | (8 if (xv < 0 and c != 0) else 0)
                    assert got == want, (float(g), i, k, float(w), got, want)
                    checked += 1
    assert checked > 1000 and skipped < checked // 100


@pytest.mark.parametrize("g_exp", [-3, 0, 5])
def test_nvfp4_quant_round_trip(g_exp):
    """Decode then requantise: a block whose values are e2m1(q) * e4m3(c) / g,
    with one element of magnitude 6 * e4m3(c) / g, quantises back to exactly
    the codes q and the scale c (g a power of two keeps everything exact).
    Code 8 (-0) comes back as 0."""
    r = inputs.rng(12345, 33 + g_exp)
    g = 2.0 ** g_exp
    e2 = _e2m1_table()
    e4 = _e4m3_table()
    R, K = 40, 64
    qs = r.integers(0, 16, size=(R, K))
    qs[:, ::16] = np.where(r.integers(0, 2, size=(R, K // 16)), 7, 15)  # |code| 6 in every block
    cs = r.integers(1, 127, size=(R, K // 16))
    cs[0, :] = [1, 8, 56, 126]  # smallest subnormal, smallest normal, 1.0, 448
    vals = np.empty((R, K))
    for i in range(R):
        for k in range(K):
            mag = e2[qs[i, k] & 7] * e4[cs[i, k // 16]] / g
            vals[i, k] = -mag if qs[i, k] & 8 else mag
    xb = bits(vals)
    assert np.array_equal(inputs.bf16_bits_to_f32(xb).astype(np.float64), vals)
    q, s = oracle.nvfp4_quant(xb, g)
    assert np.array_equal(s, cs.astype(np.uint8))
    want = np.where(qs == 8, 0, qs)
    assert np.array_equal(q & 15, want[:, 0::2]) and np.array_equal(q >> 4, want[:, 1::2])


def test_nvfp4_quant_pow2_scaling_rows_and_zero():
    x = inputs.randn_bf16((9, 128), 1.0, tag=(34,))
    xf = inputs.bf16_bits_to_f32(x)
    g = np.float32(448 * 6 / np.abs(xf).max())
    q, s = oracle.nvfp4_quant(x, g)
    # x * 2^p with g * 2^-p: every fp32 step is scaled exactly, codes unchanged
    for p in (-4, 3):
        q2, s2 = oracle.nvfp4_quant(bits(xf.astype(np.float64) * 2.0 ** p), g * np.float32(2.0 ** -p))
        assert np.array_equal(q, q2) and np.array_equal(s, s2), p
    # each row alone, and the rows reversed
    for i in range(9):
        qi, si = oracle.nvfp4_quant(x[i:i + 1], g)
        assert np.array_equal(qi[0], q[i]) and np.array_equal(si[0], s[i])
    qr, sr = oracle.nvfp4_quant(x[::-1].copy(), g)
    assert np.array_equal(qr, q[::-1]) and np.array_equal(sr, s[::-1])
    # a zero row gives zero bytes; negative zero gives code 0, not 8
    z = np.zeros((1, 32), np.uint16)
    z[0, 5] = 0x8000
    qz, sz = oracle.nvfp4_quant(z, 3.0)
    assert not qz.any() and not sz.any()


# ---------------------------------------------------------------- reduction of partials + RMSNorm
#
# oracle.reduce_rmsnorm: R = residual + sum_p P_p, Y = RMSNorm(R) (the
# all-reduce + RMSNorm pair of the vLLM PR #51292 page, section "Purpose").

@pytest.mark.parametrize("name", ["reduce_rms_two", "reduce_rms_res"])
def test_reduce_rmsnorm_worked_examples(name):
    args, rhs = WORKED[name]
    P = np.stack([bits([[float(v) for v in part.split(",")]]) for part in args["P"].split("|")])
    res = None if args["res"] == "none" else bits([[float(v) for v in args["res"].split(",")]])
    gam = bits([float(v) for v in args["gamma"].split(",")])
    want = dict(tok.split("=", 1) for tok in rhs.split())
    R, SR, Y, SY = oracle.reduce_rmsnorm(P, gam, float(args["eps"]), residual=res)
    assert R[0].tolist() == [float(v) for v in want["R"].split(",")]
    np.testing.assert_allclose(Y[0], [float(v) for v in want["Y"].split(",")], rtol=1e-15, atol=0)


def test_reduce_rmsnorm_integer_exact_and_order():
    """Integer partials: R equals numpy's int64 sum exactly, whatever the
    order of the partials; the residual acts as one more partial."""
    P = inputs.randint_bf16((5, 7, 64), -40, 40, tag=(40,))
    res = inputs.randint_bf16((7, 64), -40, 40, tag=(41,))
    gam = inputs.uniform_bf16((64,), 0.5, 1.5, tag=(42,))
    Pi = inputs.bf16_bits_to_f32(P).astype(np.int64)
    ri = inputs.bf16_bits_to_f32(res).astype(np.int64)
    R, SR, Y, SY = oracle.reduce_rmsnorm(P, gam, 1e-6, residual=res)
    assert np.array_equal(R, (Pi.sum(axis=0) + ri).astype(np.float64))
    assert np.array_equal(SR, (np.abs(Pi).sum(axis=0) + np.abs(ri)).astype(np.float64))
    R2, _, Y2, _ = oracle.reduce_rmsnorm(P[::-1].copy(), gam, 1e-6, residual=res)
    assert np.array_equal(R2, R) and np.array_equal(Y2, Y)
    R3, _, Y3, _ = oracle.reduce_rmsnorm(np.concatenate([res[None], P]), gam, 1e-6)
    assert np.array_equal(R3, R) and np.array_equal(Y3, Y)


def test_reduce_rmsnorm_single_partial_is_rmsnorm():
    """One partial and no residual reduces to RMSNorm of that partial, and the
    normalisation of R is RMSNorm's closed form (zero row -> 0)."""
    X = inputs.randn_bf16((9, 512), tag=(43,))
    X[4] = 0
    gam = inputs.uniform_bf16((512,), 0.5, 1.5, tag=(44,))
    R, SR, Y, SY = oracle.reduce_rmsnorm(X[None], gam, 1e-6)
    assert np.array_equal(R, inputs.bf16_bits_to_f32(X).astype(np.float64))
    assert np.array_equal(Y, oracle.rmsnorm(X, gam, 1e-6))
    assert not Y[4].any()
    # SY = |gamma| * SR / rms: with one partial SR = |x|, so SY = |Y|
    np.testing.assert_allclose(SY, np.abs(Y), rtol=1e-15, atol=0)


# ---------------------------------------------------------------- grouped (MoE) GEMM

def test_grouped_gemm_worked_example():
    args, rhs = WORKED["grouped_two_experts"]
    A = bits(_parse_matrix(args["A"]))
    W = np.stack([bits(_parse_matrix(w)) for w in args["W"].split("|")])
    off = [int(v) for v in args["off"].split(",")]
    y, s = oracle.grouped_gemm(A, W, off)
    assert y.tolist() == _parse_matrix(rhs)


def test_grouped_gemm_integer_exact_empty_groups_and_single_expert():
    """Integer inputs against numpy int64 per-expert matmuls, with empty
    experts; one expert covering every row is the plain GEMM."""
    T, N, K = 40, 24, 64
    off = [0, 0, 7, 7, 30, 40]          # experts 0 and 2 empty
    E = len(off) - 1
    A = inputs.randint_bf16((T, K), -3, 3, tag=(60,))
    W = inputs.randint_bf16((E, N, K), -3, 3, tag=(61,))
    Ai = inputs.bf16_bits_to_f32(A).astype(np.int64)
    Wi = inputs.bf16_bits_to_f32(W).astype(np.int64)
    y, s = oracle.grouped_gemm(A, W, off)
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        assert np.array_equal(y[rows], (Ai[rows] @ Wi[e].T).astype(np.float64))
        assert np.array_equal(s[rows], (np.abs(Ai[rows]) @ np.abs(Wi[e]).T).astype(np.float64))
    y1, s1 = oracle.grouped_gemm(A, W[3:4], [0, T])
    g, gs = oracle.gemm(A, W[3])
    assert np.array_equal(y1, g) and np.array_equal(s1, gs)


# ---------------------------------------------------------------- MLA decode attention

@pytest.mark.parametrize("name", ["attn_uniform", "attn_two"])
def test_mla_decode_worked_examples(name):
    args, rhs = WORKED[name]
    q = bits([[[float(v) for v in args["q"].split(",")]]])
    kv = bits([_parse_matrix(args["kv"])])
    o, s = oracle.mla_decode(q, kv, [kv.shape[1]], float(args["scale"]), int(args["Dv"]))
    assert math.isclose(o[0, 0, 0], float(rhs), rel_tol=1e-15)


def test_mla_decode_closed_forms_and_bruteforce():
    """One token: o = v exactly.  Identical keys: o = mean of the values.
    Token order does not matter.  Against a direct numpy softmax in fp64 on
    a small random case.  A zero-length request gives zeros."""
    r = inputs.rng(12345, 70)
    H, Dqk, Dv, L = 3, 40, 24, 9
    q = inputs.randn_bf16((2, H, Dqk), tag=(71,))
    kv = inputs.randn_bf16((2, L, Dqk), tag=(72,))
    qf = inputs.bf16_bits_to_f32(q).astype(np.float64)
    kvf = inputs.bf16_bits_to_f32(kv).astype(np.float64)
    scale = 0.125
    o, s = oracle.mla_decode(q, kv, [L, 1], scale, Dv)
    # request 1 has a single token: o = v_0 exactly, for every head
    assert np.array_equal(o[1], np.broadcast_to(kvf[1, 0, :Dv], (H, Dv)))
    # request 0 against numpy
    sc = scale * np.einsum("hd,td->ht", qf[0], kvf[0])
    p = np.exp(sc - sc.max(axis=1, keepdims=True))
    ref = (p @ kvf[0, :, :Dv]) / p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(o[0], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s[0], (p @ np.abs(kvf[0, :, :Dv])) / p.sum(axis=1, keepdims=True),
                               rtol=1e-12, atol=1e-12)
    # token order
    perm = r.permutation(L)
    o2, _ = oracle.mla_decode(q, kv[:, perm], [L, 1], scale, Dv)
    np.testing.assert_allclose(o2[0], o[0], rtol=1e-12, atol=1e-13)
    # identical keys: uniform weights, o = mean of the values
    kv_same = kv.copy()
    kv_same[0, :, Dv:] = kv[0, 0, Dv:]
    kv_same[0, :, :Dv] = 0
    kv_same[0, :, :Dv] = inputs.randint_bf16((L, Dv), -8, 8, tag=(73,))
    qz = q.copy()
    qz[0, :, :Dv] = 0            # scores then depend on the shared components only
    o3, _ = oracle.mla_decode(qz, kv_same, [L, 1], scale, Dv)
    mean = inputs.bf16_bits_to_f32(kv_same[0, :, :Dv]).astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(o3[0], np.broadcast_to(mean, (H, Dv)), rtol=1e-13, atol=1e-13)
    # empty request
    o4, s4 = oracle.mla_decode(q, kv, [0, 1], scale, Dv)
    assert not o4[0].any() and not s4[0].any()
