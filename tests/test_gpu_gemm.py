"""GPU parity and batch-invariance tests of bi_gemm (through the C ABI).

Parity: the HIP result against the fp64 oracle, element by element, within
|y - y_ref| <= ulp_bf16(y_ref) + 1e-3 * sum_k |a_k b_k|; bit-exact where the
inputs make every fp32 partial sum exact (small integers).
Invariance (bitwise, GPU against GPU): every M of a sweep against the largest
M (prefix rows), singletons, row permutations, gathered subsets at shifted
base addresses, 8 repeated runs, and persistent-grid overrides.
"""
import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_bi_amd import inputs
from invariant_deterministic_bi_amd import binding as B
from harness import assert_within_tol, rne_bf16_of_exact, bf16_to_f64
from gpu_util import dev, host, note, loaded_hip_runtimes

pytestmark = pytest.mark.gpu


def gemm(A, Bw, **kw):
    return B.bi_gemm(A, Bw, **kw)


def test_one_hip_runtime_and_torch_stream():
    a = dev(inputs.randn_bf16((4, 64), tag=(900,)))
    b = dev(inputs.randn_bf16((16, 64), tag=(901,)))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = gemm(a, b, stream=s)
    s.synchronize()
    libs = loaded_hip_runtimes()
    assert len(libs) == 1, libs
    ref, _ = oracle.gemm(host(a), host(b))
    assert np.abs(bf16_to_f64(host(y)) - ref).max() < 1e-1


def test_tiny_config_parity_and_invariance():
    """A[M,512] . B[256,512]^T, N(0,1) inputs, M in {1,3,7,16,64}."""
    K, N = 512, 256
    A = inputs.randn_bf16((64, K), tag=(1,))
    W = inputs.randn_bf16((N, K), tag=(2,))
    ref, s = oracle.gemm(A, W)
    Ad, Wd = dev(A), dev(W)
    note("gemm tiny M=64")
    y64 = host(gemm(Ad, Wd))
    assert_within_tol(y64, ref, s, "tiny M=64")
    for M in (1, 3, 7, 16):
        note(f"gemm tiny M={M}")
        yM = host(gemm(Ad[:M], Wd))
        assert np.array_equal(yM, y64[:M]), f"prefix rows differ at M={M}"
    for i in range(64):
        yi = host(gemm(Ad[i:i + 1], Wd))
        assert np.array_equal(yi[0], y64[i]), f"row {i} differs between M=1 and M=64"


@pytest.mark.parametrize("M,N,K", [(129, 200, 544), (7, 4096, 4096), (64, 6144, 4096),
                                   (33, 4096, 12288), (300, 256, 512)])
def test_integer_exact(M, N, K):
    """Entries in {-3..3}: every partial sum is an exact fp32 integer, so the
    output must be bf16_rne(exact sum) bit for bit (sums above 256 exercise
    the ties of round-to-nearest-even)."""
    A = inputs.randint_bf16((M, K), -3, 3, tag=(10, M, N, K))
    W = inputs.randint_bf16((N, K), -3, 3, tag=(11, M, N, K))
    ref, _ = oracle.gemm(A, W)
    note(f"gemm integer M={M} N={N} K={K}")
    y = host(gemm(dev(A), dev(W)))
    assert np.array_equal(y, rne_bf16_of_exact(ref))


def test_rne_ties():
    """Row sums that sit exactly halfway between two bf16 values."""
    K = 1024
    sums = np.array([257, 259, 261, 263, -257, -259, 514, 518, 522, -514, 1028, 1036, 1, 0, 255, 511])
    A = np.zeros((len(sums), K))
    for i, v in enumerate(sums):     # spread |v| over ones, sign on all of them
        n = abs(int(v))
        A[i, :min(n, K)] = np.sign(v)
        if n > K:
            A[i, :n - K] = 2 * np.sign(v)
    W = np.ones((16, K))
    Ab, Wb = inputs.to_bf16_bits(A), inputs.to_bf16_bits(W)
    ref, _ = oracle.gemm(Ab, Wb)
    note("gemm rne ties")
    y = host(gemm(dev(Ab), dev(Wb)))
    assert np.array_equal(y, rne_bf16_of_exact(ref))


def test_ragged_parity_and_tails():
    M, N, K = 129, 200, 544          # tails in every dimension
    A = inputs.randn_bf16((M, K), tag=(20,))
    W = inputs.randn_bf16((N, K), tag=(21,))
    ref, s = oracle.gemm(A, W)
    note("gemm ragged 129x200x544")
    y = host(gemm(dev(A), dev(W)))
    assert_within_tol(y, ref, s, "ragged")


def test_identity_and_scaling():
    for K in (512, 4096):
        A = inputs.randn_bf16((37, K), tag=(30, K))
        I = inputs.to_bf16_bits(np.eye(K))
        note(f"gemm identity K={K}")
        y = host(gemm(dev(A), dev(I)))
        assert np.array_equal(y, A)
    A = inputs.randn_bf16((50, 1024), tag=(31,))
    W = inputs.randn_bf16((384, 1024), tag=(32,))
    Ad, Wd = dev(A), dev(W)
    y = host(gemm(Ad, Wd))
    for p in (-3, 4):
        note(f"gemm scale 2^{p}")
        y2 = host(gemm(Ad * (2.0 ** p), Wd))
        assert np.array_equal(bf16_to_f64(y2), bf16_to_f64(y) * 2.0 ** p)


QWEN = [(6144, 4096, 2048), (4096, 4096, 2048), (24576, 4096, 2048), (4096, 12288, 8192)]


@pytest.mark.parametrize("N,K,Mmax", QWEN)
def test_linear_shapes_sweep(N, K, Mmax):
    """Qwen3-8B-shaped linears: parity on sampled rows at M_max, and every M
    of the sweep (powers of two, plus 7, 129, 1000 for the long-K case)
    bitwise equal to the prefix of the M_max result."""
    A = inputs.randn_bf16((Mmax, K), 1.0, tag=(40, N, K))
    W = inputs.randn_bf16((N, K), 0.02, tag=(41, N, K))
    Ad, Wd = dev(A), dev(W)
    note(f"gemm N={N} K={K} M={Mmax}")
    yfull = host(gemm(Ad, Wd))
    rows = np.unique(np.concatenate([[0, 1, Mmax - 1], inputs.rng(12345, 42, N).integers(0, Mmax, 5)]))
    ref, s = oracle.gemm(A, W, rows=rows)
    assert_within_tol(yfull[rows], ref, s, f"N={N} K={K} sampled rows")
    Ms = [1 << i for i in range(Mmax.bit_length()) if (1 << i) < Mmax]
    if K == 12288:
        Ms += [7, 129, 1000]
    for M in Ms:
        note(f"gemm N={N} K={K} prefix M={M}")
        y = host(gemm(Ad[:M], Wd))
        assert np.array_equal(y, yfull[:M]), f"M={M} prefix differs"
    # small-M parity directly as well
    ref1, s1 = oracle.gemm(A[:4], W)
    assert_within_tol(yfull[:4], ref1, s1, f"N={N} K={K} rows 0..3")


def test_permutations_subsets_repeats_grid():
    N, K, M = 4096, 4096, 512
    A = inputs.randn_bf16((M, K), tag=(50,))
    W = inputs.randn_bf16((N, K), 0.02, tag=(51,))
    Ad, Wd = dev(A), dev(W)
    note("gemm invariance base")
    y = host(gemm(Ad, Wd))
    g = inputs.rng(12345, 52)
    for trial in range(2):
        perm = g.permutation(M)
        note(f"gemm permutation {trial}")
        yp = host(gemm(Ad[torch.from_numpy(perm).cuda()].contiguous(), Wd))
        assert np.array_equal(yp, y[perm])
    perm = g.permutation(M)[:77]           # odd M
    yp = host(gemm(Ad[torch.from_numpy(perm).cuda()].contiguous(), Wd))
    assert np.array_equal(yp, y[perm])
    for off in (8, 24, 1000):              # subsets in fresh buffers at shifted bases
        sub = np.sort(g.choice(M, size=45, replace=False))
        buf = torch.zeros((off + 45 * K,), dtype=torch.bfloat16, device="cuda")
        view = buf[off:].view(45, K)
        view.copy_(Ad[torch.from_numpy(sub).cuda()])
        note(f"gemm subset off={off}")
        ys = host(gemm(view, Wd))
        assert np.array_equal(ys, y[sub])
    outs = set()
    for r in range(8):
        note(f"gemm repeat {r}")
        outs.add(host(gemm(Ad, Wd)).tobytes())
    assert len(outs) == 1, f"{len(outs)} distinct outputs over 8 runs"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for mw in (1, 7, cus, 4 * cus):
        note(f"gemm grid override {mw}")
        yg = host(gemm(Ad, Wd, max_workgroups=mw))
        assert np.array_equal(yg, y), f"grid {mw} differs"


def test_empty_and_strided():
    A = inputs.randn_bf16((16, 520), tag=(60,))
    W = inputs.randn_bf16((136, 520), tag=(61,))
    Ad, Wd = dev(A), dev(W)
    y0 = torch.empty((0, 136), dtype=torch.bfloat16, device="cuda")
    B.bi_gemm(Ad[:0], Wd, y0)
    # strided views: K=512 inside rows of 520
    y = host(gemm(Ad[:, :512], Wd[:, :512]))
    ref, s = oracle.gemm(A[:, :512], W[:, :512])
    assert_within_tol(y, ref, s, "strided")
    # output with a leading dimension larger than N
    ybig = torch.zeros((16, 144), dtype=torch.bfloat16, device="cuda")
    B.bi_gemm(Ad[:, :512], Wd[:, :512], ybig[:, :136])
    yb = host(ybig)
    assert np.array_equal(yb[:, :136], y)
    assert not yb[:, 136:].any()


def test_every_tile_shape_gives_the_same_bits():
    """The tile shape only decides which lane and workgroup computes an
    output: forcing each compiled shape must reproduce the plan's bits."""
    shapes = B.tile_shapes()
    assert len(shapes) >= 4
    for (M, N, K) in [(300, 4096, 4096), (5, 6144, 4096), (77, 200, 544)]:
        A = inputs.randn_bf16((M, K), tag=(70, M, N))
        W = inputs.randn_bf16((N, K), 0.02, tag=(71, M, N))
        Ad, Wd = dev(A), dev(W)
        y = host(gemm(Ad, Wd))
        for v in range(1, len(shapes) + 1):
            note(f"gemm tile variant {v} M={M} N={N} K={K}")
            yv = host(gemm(Ad, Wd, tile_variant=v))
            assert np.array_equal(yv, y), f"tile variant {v} ({shapes[v - 1]}) differs"
    with pytest.raises(B.BiError):
        gemm(Ad, Wd, tile_variant=len(shapes) + 1)


@pytest.mark.parametrize("pp,classic,bn", [(14, 13, 256), (18, 17, 192), (19, 10, 128)])
def test_pingpong_schedule_matches_classic_schedule(pp, classic, bn):
    """The ping-pong kernels (256 x 256: tile variant 14; 256 x 192: 18;
    256 x 128: 19) against the classic schedule of the same shape (13; 17;
    10): ragged M and N,
    K % 64 == 32, several grid caps, each run repeated (a phase-ordering race
    would show as a rare mismatch)."""
    shapes = B.tile_shapes()
    assert shapes[pp - 1]["bm"] == 256 and shapes[pp - 1]["bn"] == bn
    assert shapes[classic - 1]["bm"] == 256 and shapes[classic - 1]["bn"] == bn
    for (M, N, K) in [(1000, 2600, 4160), (513, 1300, 2080), (2048, 6144, 4096), (77, 200, 544)]:
        A = inputs.randn_bf16((M, K), tag=(75, M, N))
        W = inputs.randn_bf16((N, K), 0.02, tag=(76, M, N))
        Ad, Wd = dev(A), dev(W)
        y = host(gemm(Ad, Wd, tile_variant=classic))
        for mw in (0, 7, 64):
            for rep in range(2):
                note(f"pingpong {bn} M={M} N={N} K={K} grid cap {mw} rep {rep}")
                assert np.array_equal(host(gemm(Ad, Wd, tile_variant=pp, max_workgroups=mw)), y), (M, N, K, mw, rep)
        if M == 2048:
            ref, s = oracle.gemm(A[[0, 511, 2047]], W)
            assert_within_tol(host(gemm(Ad, Wd, tile_variant=pp))[[0, 511, 2047]], ref, s, "pingpong")


@pytest.mark.parametrize("N,K,fp4", [(6144, 4096, False), (8200, 2048, False), (24576, 4096, True),
                                     (6144, 4096, True), (8200, 2048, True)])
def test_chunked_a_path_matches_tiled_kernel(N, K, fp4):
    """16 < M <= 64 with A staged in LDS in K chunks (more 16-column items
    than compute units; bf16 and NVFP4 weights, ragged N), and 64 < M <= 128
    (eight row blocks) for an NVFP4 weight with at least four items per
    compute unit: every M in {17, 20, 32, 33, 48, 63, 64} (and {65, 100,
    127, 128}) bitwise equal to the forced tiled kernel and to the full
    batch, under wavefront caps {1, 7, #CU} and pipeline depths {1, 2, 4, 8};
    parity with the oracle."""
    plan = B.plan_regimes(B.BI_OP_NVFP4_GEMM if fp4 else B.BI_OP_GEMM, N, K)
    chunked = [r for r in plan if r["kind"] == "stream_a_chunks"]
    assert chunked and chunked[0]["m_min"] == 17, plan
    wide = chunked[-1]["m_max"] >= 128
    assert wide == (fp4 and N == 24576), plan
    Mmax = 128 if wide else 64
    A = inputs.randn_bf16((Mmax, K), tag=(90, N, K))
    if fp4:
        x = inputs.rng(12345, 91, N, K).standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
        g = inputs.nvfp4_global_scale(x)
        W, Ws = inputs.nvfp4_quantize(x, g)
        alpha = float(np.float32(1.0) / g)
        Ad, Wd, Wsd = dev(A), dev(W), dev(Ws)

        def run(M, **kw):
            return host(B.bi_nvfp4_gemm(Ad[:M], Wd, Wsd, alpha, **kw))
        tiled = 13
    else:
        W = inputs.randn_bf16((N, K), 0.02, tag=(92, N, K))
        Ad, Wd = dev(A), dev(W)

        def run(M, **kw):
            return host(gemm(Ad[:M], Wd, **kw))
        tiled = 1
    note(f"chunked A N={N} K={K} fp4={fp4} M={Mmax}")
    yfull = run(Mmax)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for M in (17, 20, 32, 33, 48, 63, 64) + ((65, 100, 127, 128) if wide else ()):
        note(f"chunked A N={N} K={K} fp4={fp4} M={M}")
        y = run(M)
        assert np.array_equal(y, yfull[:M]), f"M={M} vs batch"
        assert np.array_equal(y, run(M, tile_variant=tiled)), f"M={M} vs tiled"
        for mw in (1, 7, cus):
            assert np.array_equal(run(M, max_workgroups=mw), y), (M, mw)
        for depth in (1, 2, 4, 8):
            assert np.array_equal(run(M, pipeline_depth=depth), y), (M, depth)
    rows = [0, 17, 63] + ([127] if wide else [])
    if fp4:
        ref, s = oracle.nvfp4_gemm(A[rows], None, W, Ws, alpha, K)
    else:
        ref, s = oracle.gemm(A[rows], W)
    assert_within_tol(yfull[rows], ref, s, f"chunked A N={N} K={K}")


@pytest.mark.parametrize("N,K", [(200, 544), (4100, 4128), (256, 96), (6144, 4096), (8200, 512)])
def test_small_m_path_matches_tiled_kernel(N, K):
    """M <= 64 runs the direct kernels (8- or 16-column items streamed into
    registers; A in LDS or loaded with the weight; above 16 rows, two or
    four 16-row blocks of A per weight fragment).  Their rows must be
    bitwise the tiled kernel's (forced with tile_variant) and the full-batch
    rows, for ragged N, K % 64 == 32 (the trailing zero-filled chunk), a
    strided A, capped wavefront counts and every pipeline depth; and within
    the oracle tolerance."""
    Mmax = 136
    W = inputs.randn_bf16((N, K), 0.02, tag=(951, N, K))
    Wd = dev(W)
    Ad = dev(inputs.randn_bf16((Mmax, K + 24), tag=(950, N, K)))[:, :K]   # row stride K + 24
    A = host(Ad)
    note(f"skinny N={N} K={K} full")
    yfull = host(gemm(Ad, Wd))
    for M in (1, 2, 3, 5, 8, 9, 16, 17, 31, 32, 33, 40):
        note(f"skinny N={N} K={K} M={M}")
        ys = host(gemm(Ad[:M], Wd))
        yt = host(gemm(Ad[:M], Wd, tile_variant=1))
        assert np.array_equal(ys, yt), f"skinny vs tiled, M={M}"
        assert np.array_equal(ys, yfull[:M]), f"skinny vs full batch, M={M}"
        for mw in (1, 5):
            assert np.array_equal(host(gemm(Ad[:M], Wd, max_workgroups=mw)), ys), (M, mw)
        for depth in (1, 2, 4, 32):
            assert np.array_equal(host(gemm(Ad[:M], Wd, pipeline_depth=depth)), ys), (M, depth)
    for M in (48, 64, 65, 100, 128):
        note(f"skinny N={N} K={K} M={M}")
        ys = host(gemm(Ad[:M], Wd))
        assert np.array_equal(ys, host(gemm(Ad[:M], Wd, tile_variant=1))), f"skinny vs tiled, M={M}"
        assert np.array_equal(ys, yfull[:M]), f"skinny vs full batch, M={M}"
        assert np.array_equal(host(gemm(Ad[:M], Wd, max_workgroups=3)), ys), M
    rows = [0, 4, 15]
    ref, s = oracle.gemm(A[rows], W)
    assert_within_tol(host(gemm(Ad[:16], Wd))[rows], ref, s, f"skinny N={N} K={K}")
    rows = [16, 33, 63]
    ref, s = oracle.gemm(A[rows], W)
    assert_within_tol(host(gemm(Ad[:64], Wd))[rows], ref, s, f"direct 64 rows N={N} K={K}")


@pytest.mark.parametrize("N,K", [(1000, 4160), (1000, 4096), (520, 1024)])
def test_small_m_nvfp4_path_matches_tiled_kernel(N, K):
    """The NVFP4 weight at M <= 16 (K % 128 == 0: codes and scales loaded
    into registers, transposed across lanes and decoded per lane, A in LDS;
    else the LDS-ring skinny kernel), and at 16 < M <= 64 with K % 128 == 0
    (the register kernel with two or four 16-row blocks of A), against the
    tiled kernel and the full batch (M = 80, tiled), under capped wavefront
    counts and every pipeline depth."""
    x = inputs.rng(12345, 952).standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    g = inputs.nvfp4_global_scale(x)
    Wq, Ws = inputs.nvfp4_quantize(x, g)
    alpha = float(np.float32(1.0) / g)
    A = inputs.randn_bf16((80, K), tag=(953,))
    Ad, Wqd, Wsd = dev(A), dev(Wq), dev(Ws)
    note("skinny nvfp4 full")
    yfull = host(B.bi_nvfp4_gemm(Ad, Wqd, Wsd, alpha))
    for M in (1, 2, 7, 9, 16, 17, 32, 33, 64):
        note(f"skinny nvfp4 N={N} K={K} M={M}")
        ys = host(B.bi_nvfp4_gemm(Ad[:M], Wqd, Wsd, alpha))
        yt = host(B.bi_nvfp4_gemm(Ad[:M], Wqd, Wsd, alpha, tile_variant=3))
        assert np.array_equal(ys, yt), f"skinny vs tiled, M={M}"
        assert np.array_equal(ys, yfull[:M]), f"skinny vs full batch, M={M}"
        for mw, depth in ((1, 0), (7, 0), (0, 1), (0, 2), (0, 16)):
            yo = host(B.bi_nvfp4_gemm(Ad[:M], Wqd, Wsd, alpha, max_workgroups=mw, pipeline_depth=depth))
            assert np.array_equal(yo, ys), (M, mw, depth)
    ref, s = oracle.nvfp4_gemm(A[:3], None, Wq, Ws, alpha, K)
    assert_within_tol(host(B.bi_nvfp4_gemm(Ad[:3], Wqd, Wsd, alpha)), ref, s, "skinny nvfp4")
