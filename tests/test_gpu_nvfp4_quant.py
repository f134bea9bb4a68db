"""GPU parity and invariance tests of bi_nvfp4_quant, the row-local NVFP4
activation quantiser, and of the W4A4 GEMM it feeds.  Codes and scales are
integer outputs: they must equal the oracle's bytes exactly."""
import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_bi_amd import inputs
from invariant_deterministic_bi_amd import binding as B
from harness import assert_within_tol
from gpu_util import dev, host, note
from test_oracle_pins import QUANT_EXAMPLES, bits

pytestmark = pytest.mark.gpu


def u8(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_quant(X, g, **kw):
    q, s = B.bi_nvfp4_quant(X, g, **kw)
    return u8(q), u8(s)


def global_scale(xbits):
    return inputs.nvfp4_global_scale(inputs.bf16_bits_to_f32(xbits))


@pytest.mark.parametrize("name", sorted(QUANT_EXAMPLES))
def test_quant_worked_examples(name):
    g, x, codes, scales = QUANT_EXAMPLES[name]
    note(f"nvfp4_quant example {name}")
    q, s = gpu_quant(dev(bits([x])), g)
    assert q[0].tolist() == codes.tolist() and s[0].tolist() == scales.tolist()


@pytest.mark.parametrize("M,K", [(1, 16), (3, 48), (7, 4096), (129, 4096), (64, 12288),
                                 (1000, 512), (4096, 4096)])
def test_quant_parity_and_row_invariance(M, K):
    X = inputs.randn_bf16((M, K), 1.0, tag=(200, M, K))
    g = global_scale(X)
    qo, so = oracle.nvfp4_quant(X, g)
    Xd = dev(X)
    note(f"nvfp4_quant M={M} K={K}")
    q, s = gpu_quant(Xd, g)
    assert np.array_equal(q, qo) and np.array_equal(s, so)
    # prefixes, single rows, a permutation, grid caps, repeated runs
    for m in sorted({1, 2, M // 2, M - 1} - {0}):
        qm, sm = gpu_quant(Xd[:m], g)
        assert np.array_equal(qm, q[:m]) and np.array_equal(sm, s[:m]), m
    for i in sorted({0, M // 3, M - 1}):
        qi, si = gpu_quant(Xd[i:i + 1], g)
        assert np.array_equal(qi[0], q[i]) and np.array_equal(si[0], s[i]), i
    perm = inputs.rng(12345, 201).permutation(M)
    qp, sp = gpu_quant(Xd[torch.from_numpy(perm).cuda()].contiguous(), g)
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])
    for mw in (1, 7):
        qw, sw = gpu_quant(Xd, g, max_workgroups=mw)
        assert np.array_equal(qw, q) and np.array_equal(sw, s)
    outs = {b"".join(a.tobytes() for a in gpu_quant(Xd, g)) for _ in range(8)}
    assert len(outs) == 1


def test_quant_extreme_scales_and_rows():
    """Tiny g (zero and subnormal E4M3 scales), huge g (saturation at 448 and
    6), zero rows, and rows spanning many magnitudes."""
    M, K = 16, 256
    r = inputs.rng(12345, 202)
    x = r.standard_normal((M, K)) * np.exp2(r.integers(-20, 20, size=(M, 1)))
    x[3] = 0.0
    x[5, ::3] = 0.0
    X = inputs.to_bf16_bits(x)
    Xd = dev(X)
    for g in (1e-9, 3.0e-6, 0.25, 1.0, 448.0, 1.0e9, float(global_scale(X))):
        qo, so = oracle.nvfp4_quant(X, g)
        note(f"nvfp4_quant g={g}")
        q, s = gpu_quant(Xd, g)
        assert np.array_equal(q, qo) and np.array_equal(s, so), g


def test_quant_padded_strides_leave_padding_alone():
    M, K, ldx, ldq = 9, 96, 104, 128
    X = inputs.randn_bf16((M, ldx), 1.0, tag=(203,))
    g = global_scale(X[:, :K])
    qo, so = oracle.nvfp4_quant(np.ascontiguousarray(X[:, :K]), g)
    Xd = dev(X)[:, :K]
    Qbuf = torch.full((M, ldq // 2), 0xAB, dtype=torch.uint8, device="cuda")
    Sbuf = torch.full((M, ldq // 16), 0xCD, dtype=torch.uint8, device="cuda")
    note("nvfp4_quant padded strides")
    B.bi_nvfp4_quant(Xd, g, Qbuf[:, :K // 2], Sbuf[:, :K // 16])
    q, s = u8(Qbuf), u8(Sbuf)
    assert np.array_equal(q[:, :K // 2], qo) and np.array_equal(s[:, :K // 16], so)
    assert (q[:, K // 2:] == 0xAB).all() and (s[:, K // 16:] == 0xCD).all()


def test_w4a4_gemm_from_gpu_quantised_activations():
    """bf16 activations -> bi_nvfp4_quant -> bi_nvfp4_gemm(NVFP4 A): within
    the oracle tolerance of the oracle GEMM on the oracle's codes (identical
    bytes), and each row quantised and multiplied alone equals its row in the
    batch."""
    N, K, M = 1024, 4096, 96
    w = inputs.rng(12345, 204).standard_normal((N, K)) * 0.02
    gw = inputs.nvfp4_global_scale(w)
    W, Ws = inputs.nvfp4_quantize(w, gw)
    X = inputs.randn_bf16((M, K), 1.0, tag=(205,))
    ga = global_scale(X)
    alpha = float(np.float32(1.0) / (ga * gw))
    Xd, Wd, Wsd = dev(X), dev(W), dev(Ws)
    note("w4a4 quant + gemm")
    q, s = B.bi_nvfp4_quant(Xd, ga)
    y = host(B.bi_nvfp4_gemm(q, Wd, Wsd, alpha, A_scales=s))
    qo, so = oracle.nvfp4_quant(X, ga)
    assert np.array_equal(u8(q), qo) and np.array_equal(u8(s), so)
    rows = [0, 1, 47, 95]
    ref, tol = oracle.nvfp4_gemm(qo, so, W, Ws, alpha, K, rows=rows)
    assert_within_tol(y[rows], ref, tol, "w4a4 rows")
    for i in (0, 50, 95):
        qi, si = B.bi_nvfp4_quant(Xd[i:i + 1], ga)
        yi = host(B.bi_nvfp4_gemm(qi, Wd, Wsd, alpha, A_scales=si))
        assert np.array_equal(yi[0], y[i]), i
