"""GPU parity and invariance tests of bi_grouped_gemm, the mixture-of-experts
grouped GEMM: each token's row must be bitwise bi_gemm of that row alone with
its expert's weight, whatever the other experts' group sizes."""
import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_bi_amd import inputs
from invariant_deterministic_bi_amd import binding as B
from harness import assert_within_tol, rne_bf16_of_exact
from gpu_util import dev, host, note

pytestmark = pytest.mark.gpu


def offsets_dev(off):
    return torch.tensor(off, dtype=torch.int64, device="cuda")


@pytest.mark.parametrize("E,N,K,sizes", [(8, 512, 1024, [3, 0, 40, 1, 17, 0, 300, 9]),
                                         (4, 6144, 4096, [1, 129, 0, 70]),
                                         (1, 6144, 512, [33]),
                                         (3, 200, 544, [5, 16, 1]),
                                         (64, 256, 512, [0] * 20 + [1, 2000] + [0] * 30 + [5] + [0] * 11),
                                         # the tile bands by rows per expert at N = 4096: 256 x 128,
                                         # 256 x 192, 256 x 256
                                         (4, 4096, 1024, [150, 100, 170, 180]),
                                         (4, 4096, 1024, [300, 250, 0, 650]),
                                         (2, 4096, 512, [900, 1300])])
def test_grouped_parity_and_rows_alone(E, N, K, sizes):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    T = int(off[-1])
    A = inputs.randn_bf16((T, K), 1.0, tag=(400, E, N))
    W = inputs.randn_bf16((E, N, K), 0.02, tag=(401, E, N))
    Ad, Wd = dev(A), dev(W)
    note(f"grouped E={E} N={N} K={K} T={T}")
    y = host(B.bi_grouped_gemm(Ad, Wd, offsets_dev(off)))
    rows = np.unique(np.concatenate([[0, T - 1], inputs.rng(12345, 402).integers(0, T, 6)]))
    ref, s = oracle.grouped_gemm(A, W, off)
    assert_within_tol(y[rows], ref[rows], s[rows], "grouped sampled rows")
    for e in range(E):
        t0, t1 = int(off[e]), int(off[e + 1])
        if t1 == t0:
            continue
        # the expert's rows as one GEMM, and its first and last row alone
        assert np.array_equal(host(B.bi_gemm(Ad[t0:t1], Wd[e])), y[t0:t1]), e
        for t in sorted({t0, t1 - 1}):
            assert np.array_equal(host(B.bi_gemm(Ad[t:t + 1], Wd[e])), y[t:t + 1]), (e, t)
    for mw in (1, 5):
        assert np.array_equal(host(B.bi_grouped_gemm(Ad, Wd, offsets_dev(off), max_workgroups=mw)), y)
    outs = {host(B.bi_grouped_gemm(Ad, Wd, offsets_dev(off))).tobytes() for _ in range(4)}
    assert len(outs) == 1


def test_grouped_batch_composition_invariance_and_integer_exact():
    """The same tokens routed in two batches of different composition (other
    tokens added to every expert) give the same bits; integer inputs give
    bf16_rne(exact)."""
    E, N, K = 6, 1024, 2048
    W = inputs.randint_bf16((E, N, K), -3, 3, tag=(410,))
    X = inputs.randint_bf16((64, K), -3, 3, tag=(411,))
    extra = inputs.randint_bf16((200, K), -3, 3, tag=(412,))
    expert_of = inputs.rng(12345, 413).integers(0, E, 64)
    extra_of = inputs.rng(12345, 414).integers(0, E, 200)
    Wd = dev(W)
    results = []
    for with_extra in (False, True):
        toks = list(range(64)) + (list(range(64, 264)) if with_extra else [])
        src = np.concatenate([X, extra]) if with_extra else X
        exp = np.concatenate([expert_of, extra_of]) if with_extra else expert_of
        order = sorted(toks, key=lambda t: (exp[t], t))
        A = src[order]
        sizes = np.bincount(exp[toks], minlength=E)
        off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
        note(f"grouped composition extra={with_extra}")
        y = host(B.bi_grouped_gemm(dev(A), Wd, offsets_dev(off)))
        ref, _ = oracle.grouped_gemm(A, W, off)
        assert np.array_equal(y, rne_bf16_of_exact(ref))
        pos = {t: i for i, t in enumerate(order)}
        results.append(np.stack([y[pos[t]] for t in range(64)]))
    assert np.array_equal(results[0], results[1])
