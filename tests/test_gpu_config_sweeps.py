"""GPU tests over the full configurations: every M of each sweep, every row
alone, the kernel-regime edges of each (N, K), the W4A4 (NVFP4 activations x
NVFP4 weight) product at the NVFP4 configuration's shape, and identical bits
in a fresh process.

The bitwise comparisons run on the device (torch.equal) so that thousands of
single-row calls stay cheap; parity against the fp64 oracle is checked on
rows sampled from every 256-row M-tile.
"""
import functools
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_bi_amd import inputs
from invariant_deterministic_bi_amd import binding as B
from harness import assert_within_tol
from gpu_util import dev, host, note

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@functools.lru_cache(maxsize=4)
def _nvfp4_weights(N, K, tag):
    x = inputs.rng(12345, *tag).standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    g = inputs.nvfp4_global_scale(x)
    W, Ws = inputs.nvfp4_quantize(x, g)
    return W, Ws, g


def _tile_rows(Mmax, tile=256, seed_tag=0):
    """Rows sampled from every `tile`-row M-tile: its first, its last and one
    seeded row inside it."""
    g = inputs.rng(12345, 700, seed_tag)
    rows = []
    for t0 in range(0, Mmax, tile):
        t1 = min(Mmax, t0 + tile) - 1
        rows += [t0, t1, int(g.integers(t0, t1 + 1))]
    return np.unique(np.array(rows))


def _sweep_ms(Mmax, odd=()):
    return sorted({1 << i for i in range(Mmax.bit_length()) if (1 << i) < Mmax} | set(odd))


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


# ------------------------------------------------------------ NVFP4, bf16 A


def test_nvfp4_bf16a_every_m_every_row_and_grid():
    """NVFP4 weight W[24576,4096] (N(0,0.02) quantised), bf16 A ~ N(0,1),
    M up to 4096: every power of two and 7, 129, 1000 bitwise equal to the
    M = 4096 prefix; every row alone equal to its row; grid caps {1, 7,
    #CU, 4 #CU} at M = 1000; 8 repeated runs; parity on rows of every M-tile."""
    N, K, Mmax = 24576, 4096, 4096
    W, Ws, g = _nvfp4_weights(N, K, (125,))
    alpha = float(np.float32(1.0) / g)
    A = inputs.randn_bf16((Mmax, K), tag=(126,))
    Ad, Wd, Wsd = dev(A), dev(W), dev(Ws)
    note("nvfp4 bf16-A M=4096")
    yfull = B.bi_nvfp4_gemm(Ad, Wd, Wsd, alpha)
    rows = _tile_rows(Mmax, seed_tag=1)
    ref, s = oracle.nvfp4_gemm(A, None, W, Ws, alpha, K, rows=rows)
    assert_within_tol(host(yfull)[rows], ref, s, "nvfp4 bf16-A rows of every M-tile")
    for M in _sweep_ms(Mmax, (7, 129, 1000)):
        note(f"nvfp4 bf16-A prefix M={M}")
        assert torch.equal(B.bi_nvfp4_gemm(Ad[:M], Wd, Wsd, alpha), yfull[:M]), M
    note("nvfp4 bf16-A every row alone")
    ys = torch.empty_like(yfull)
    for i in range(Mmax):
        B.bi_nvfp4_gemm(Ad[i:i + 1], Wd, Wsd, alpha, ys[i:i + 1])
    assert torch.equal(ys, yfull)
    for mw in (1, 7, _cus(), 4 * _cus()):
        note(f"nvfp4 bf16-A grid cap {mw} at M=1000")
        assert torch.equal(B.bi_nvfp4_gemm(Ad[:1000], Wd, Wsd, alpha, max_workgroups=mw), yfull[:1000]), mw
    note("nvfp4 bf16-A 8 repeats")
    for r in range(8):
        assert torch.equal(B.bi_nvfp4_gemm(Ad, Wd, Wsd, alpha), yfull), r


# ------------------------------------------------------------ W4A4


def test_w4a4_config_parity_and_invariance():
    """W4A4 at W[24576,4096]: A ~ N(0,1) quantised per row by bi_nvfp4_quant
    with the global scale of the whole M = 4096 batch (the activation
    quantiser of the NVFP4 summary page's unit test).  The codes agree with
    the oracle's on rows of every M-tile; the product is within tolerance of
    the oracle there; every power of two and 7, 129, 1000 is bitwise the
    M = 4096 prefix; rows 0, 7, 100 and 4095 quantised alone give the same
    codes and the same output row; every row alone equals its row; 8 repeats
    agree."""
    N, K, Mmax = 24576, 4096, 4096
    W, Ws, gw = _nvfp4_weights(N, K, (125,))
    X = inputs.randn_bf16((Mmax, K), tag=(160,))
    ga = inputs.nvfp4_global_scale(inputs.bf16_bits_to_f32(X))
    alpha = float(np.float32(1.0) / (np.float32(ga) * np.float32(gw)))
    Xd, Wd, Wsd = dev(X), dev(W), dev(Ws)
    note("w4a4 quantise M=4096")
    Aq, Aqs = B.bi_nvfp4_quant(Xd, ga)
    torch.cuda.synchronize()
    Aqh, Aqsh = Aq.cpu().numpy(), Aqs.cpu().numpy()
    rows = _tile_rows(Mmax, seed_tag=2)
    qo, so = oracle.nvfp4_quant(X[rows], ga)
    assert np.array_equal(Aqh[rows], qo) and np.array_equal(Aqsh[rows], so), "quantiser codes"
    note("w4a4 gemm M=4096")
    yfull = B.bi_nvfp4_gemm(Aq, Wd, Wsd, alpha, A_scales=Aqs)
    ref, s = oracle.nvfp4_gemm(Aqh, Aqsh, W, Ws, alpha, K, rows=rows)
    assert_within_tol(host(yfull)[rows], ref, s, "w4a4 rows of every M-tile")
    for M in _sweep_ms(Mmax, (7, 129, 1000)):
        note(f"w4a4 prefix M={M}")
        assert torch.equal(B.bi_nvfp4_gemm(Aq[:M], Wd, Wsd, alpha, A_scales=Aqs[:M]), yfull[:M]), M
    for i in (0, 7, 100, Mmax - 1):
        note(f"w4a4 row {i} quantised alone")
        qi, si = B.bi_nvfp4_quant(Xd[i:i + 1], ga)
        assert torch.equal(qi[0], Aq[i]) and torch.equal(si[0], Aqs[i]), i
        assert torch.equal(B.bi_nvfp4_gemm(qi, Wd, Wsd, alpha, A_scales=si)[0], yfull[i]), i
    note("w4a4 every row alone")
    ys = torch.empty_like(yfull)
    for i in range(Mmax):
        B.bi_nvfp4_gemm(Aq[i:i + 1], Wd, Wsd, alpha, ys[i:i + 1], A_scales=Aqs[i:i + 1])
    assert torch.equal(ys, yfull)
    note("w4a4 8 repeats")
    for r in range(8):
        assert torch.equal(B.bi_nvfp4_gemm(Aq, Wd, Wsd, alpha, A_scales=Aqs), yfull), r


def test_w4a4_config_tile_variants_and_grid():
    """W4A4 at W[24576,4096], M = 1000 (a ragged last M-tile): every compiled
    tile shape forced (the 256 x 256 shapes 0 and 12 among them; 12 is the
    plan's) and the grid caps {1, 7, #CU, 4 #CU} give the plan's bits."""
    N, K, M = 24576, 4096, 1000
    W, Ws, gw = _nvfp4_weights(N, K, (125,))
    X = inputs.randn_bf16((M, K), tag=(161,))
    ga = inputs.nvfp4_global_scale(inputs.bf16_bits_to_f32(X))
    alpha = float(np.float32(1.0) / (np.float32(ga) * np.float32(gw)))
    Wd, Wsd = dev(W), dev(Ws)
    Aq, Aqs = B.bi_nvfp4_quant(dev(X), ga)
    note("w4a4 M=1000 plan")
    y = B.bi_nvfp4_gemm(Aq, Wd, Wsd, alpha, A_scales=Aqs)
    plan = B.plan_query(B.BI_OP_NVFP4_GEMM, N, K)
    assert (plan["bm"], plan["bn"]) == (256, 256)
    for v in range(1, len(B.tile_shapes()) + 1):
        note(f"w4a4 M=1000 tile variant {v}")
        assert torch.equal(B.bi_nvfp4_gemm(Aq, Wd, Wsd, alpha, A_scales=Aqs, tile_variant=v), y), v
    for mw in (1, 7, _cus(), 4 * _cus()):
        note(f"w4a4 M=1000 grid cap {mw}")
        assert torch.equal(B.bi_nvfp4_gemm(Aq, Wd, Wsd, alpha, A_scales=Aqs, max_workgroups=mw), y), mw
    ref, s = oracle.nvfp4_gemm(Aq.cpu().numpy()[[0, 999]], Aqs.cpu().numpy()[[0, 999]], W, Ws, alpha, K)
    assert_within_tol(host(y)[[0, 999]], ref, s, "w4a4 M=1000")


# ------------------------------------------------------------ regime edges

def _regime_ms(op, N, K, a_fmt=B.BI_A_BF16, mmax=4200):
    """M values on both sides of every edge bi_plan_regimes lists for (op,
    N, K) on this device (the kernel or tile shape changes there), plus 1
    and the 256-row M-tile edges."""
    ms = {1, 2, 255, 256, 257}
    for r in B.plan_regimes(op, N, K, a_fmt):
        ms |= {r["m_min"], r["m_min"] + 1, r["m_max"], r["m_max"] + 1}
    return sorted(m for m in ms if 1 <= m <= mmax)


CONFIG_NK = [(256, 512), (6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288)]


@pytest.mark.parametrize("N,K", CONFIG_NK)
def test_regime_edges_bf16(N, K):
    """Every configuration's (N, K), M walked across every edge of the
    kernel and tile-shape choice that bi_plan_regimes lists (up to 4200
    rows, past the last edge): each M's rows are bitwise the forced tiled
    kernel's (tile shape 0, 256 x 256) and the M = 4200 batch's prefix."""
    Mmax = 4200
    A = inputs.randn_bf16((Mmax, K), tag=(710, N, K))
    W = inputs.randn_bf16((N, K), 0.02, tag=(711, N, K))
    Ad, Wd = dev(A), dev(W)
    note(f"regime edges bf16 N={N} K={K} M={Mmax}")
    yfull = B.bi_gemm(Ad, Wd)
    for M in _regime_ms(B.BI_OP_GEMM, N, K):
        note(f"regime edges bf16 N={N} K={K} M={M}")
        y = B.bi_gemm(Ad[:M], Wd)
        assert torch.equal(y, yfull[:M]), f"M={M} vs batch"
        assert torch.equal(y, B.bi_gemm(Ad[:M], Wd, tile_variant=1)), f"M={M} vs tiled"
    rows = [0, 17, 299, 2100, Mmax - 1]
    ref, s = oracle.gemm(A[rows], W)
    assert_within_tol(host(yfull)[rows], ref, s, f"N={N} K={K}")


@pytest.mark.parametrize("a_fp4", [False, True], ids=["bf16A", "w4a4"])
def test_regime_edges_nvfp4(a_fp4):
    """The NVFP4 configuration's (24576, 4096), bf16 or NVFP4 A: M across
    every edge bi_plan_regimes lists (up to 4200 rows), bitwise equal to the
    forced 256 x 256 tiled kernel (classic schedule) and the batch prefix."""
    N, K, Mmax = 24576, 4096, 4200
    W, Ws, g = _nvfp4_weights(N, K, (125,))
    alpha = float(np.float32(1.0) / g)
    A = inputs.randn_bf16((Mmax, K), tag=(712,))
    Ad, Wd, Wsd = dev(A), dev(W), dev(Ws)
    if a_fp4:
        Aq, Aqs = B.bi_nvfp4_quant(Ad, 1.0)

        def run(M, **kw):
            return B.bi_nvfp4_gemm(Aq[:M], Wd, Wsd, alpha, A_scales=Aqs[:M], **kw)
    else:
        def run(M, **kw):
            return B.bi_nvfp4_gemm(Ad[:M], Wd, Wsd, alpha, **kw)
    tag = "w4a4" if a_fp4 else "nvfp4"
    note(f"regime edges {tag} M={Mmax}")
    yfull = run(Mmax)
    for M in _regime_ms(B.BI_OP_NVFP4_GEMM, N, K, B.BI_A_NVFP4 if a_fp4 else B.BI_A_BF16):
        note(f"regime edges {tag} M={M}")
        y = run(M)
        assert torch.equal(y, yfull[:M]), f"M={M} vs batch"
        assert torch.equal(y, run(M, tile_variant=13)), f"M={M} vs tiled"


# ------------------------------------------------------------ every row alone

@pytest.mark.parametrize("N,K,Mmax", [(6144, 4096, 2048), (4096, 4096, 2048), (24576, 4096, 2048),
                                      (4096, 12288, 8192)])
def test_every_row_alone_linears(N, K, Mmax):
    """Every row of the Qwen3-8B-shaped linears computed alone (M = 1) is
    bitwise its row of the M_max batch (the row-by-row check of the NVFP4
    summary page's unit test); parity on rows of every 256-row M-tile."""
    A = inputs.randn_bf16((Mmax, K), 1.0, tag=(40, N, K))
    W = inputs.randn_bf16((N, K), 0.02, tag=(41, N, K))
    Ad, Wd = dev(A), dev(W)
    note(f"every row alone N={N} K={K} M={Mmax}")
    yfull = B.bi_gemm(Ad, Wd)
    ys = torch.empty_like(yfull)
    for i in range(Mmax):
        B.bi_gemm(Ad[i:i + 1], Wd, ys[i:i + 1])
    assert torch.equal(ys, yfull)
    rows = _tile_rows(Mmax, seed_tag=N + K)
    ref, s = oracle.gemm(A, W, rows=rows)
    assert_within_tol(host(yfull)[rows], ref, s, f"N={N} K={K} rows of every M-tile")


def test_every_row_alone_rmsnorm_and_bmm():
    """RMSNorm over hidden 4096 (M = 2048) and the MLA-absorbed BMM (128
    heads, M = 1024): every row alone, and every power-of-two prefix."""
    H, Mmax = 4096, 2048
    X = dev(inputs.randn_bf16((Mmax, H), tag=(720,)))
    gam = dev(inputs.uniform_bf16((H,), 0.5, 1.5, tag=(721,)))
    note("rmsnorm every row alone")
    y = B.bi_rmsnorm(X, gam, 1e-6)
    ys = torch.empty_like(y)
    for i in range(Mmax):
        B.bi_rmsnorm(X[i:i + 1], gam, 1e-6, ys[i:i + 1])
    assert torch.equal(ys, y)
    for M in _sweep_ms(Mmax):
        assert torch.equal(B.bi_rmsnorm(X[:M], gam, 1e-6), y[:M]), M
    Hh, Mb = 128, 1024
    A = dev(inputs.randn_bf16((Hh, Mb, 128), tag=(722,)))
    Wm = dev(inputs.randn_bf16((Hh, 128, 512), tag=(723,)))
    note("bmm every row alone")
    yb = B.bi_bmm(A, Wm)
    ysb = torch.empty_like(yb)
    for i in range(Mb):
        B.bi_bmm(A[:, i:i + 1], Wm, ysb[:, i:i + 1])
    assert torch.equal(ysb, yb)
    for M in _sweep_ms(Mb):
        assert torch.equal(B.bi_bmm(A[:, :M], Wm), yb[:, :M]), M


# ------------------------------------------------------------ fresh process

def test_fresh_process_gives_the_same_bits():
    """The outputs of one process equal those of a fresh one (the 8-runs
    check of the fuse_allreduce_rms PR page's test plan, across processes):
    a child process computes the same seeded cases and reports SHA-256
    digests of the output bytes."""
    import fresh_process_cases as fpc
    note("fresh process: in-process digests")
    mine = fpc.digests()
    note("fresh process: child")
    env = dict(os.environ)
    r = subprocess.run([sys.executable, os.path.join(HERE, "fresh_process_cases.py")], capture_output=True,
                       text=True, timeout=300, env=env, cwd=os.path.dirname(HERE))
    assert r.returncode == 0, r.stderr[-2000:]
    theirs = json.loads(r.stdout.strip().splitlines()[-1])
    assert theirs == mine
