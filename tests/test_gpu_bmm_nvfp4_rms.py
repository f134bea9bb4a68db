"""GPU parity and invariance tests of bi_bmm, bi_nvfp4_gemm and bi_rmsnorm."""
import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_bi_amd import inputs
from invariant_deterministic_bi_amd import binding as B
from harness import assert_within_tol, rne_bf16_of_exact, bf16_to_f64, ulp_bf16
from gpu_util import dev, host, note

pytestmark = pytest.mark.gpu

# ----------------------------------------------------------------- BMM


def test_bmm_mla_shape_parity_and_invariance():
    """128 heads, per head A[M,128] . B[128,512]; M in {1,16,128,1024}."""
    H, K, N, Mmax = 128, 128, 512, 1024
    A = inputs.randn_bf16((H, Mmax, K), tag=(100,))
    W = inputs.randn_bf16((H, K, N), tag=(101,))
    Ad, Wd = dev(A), dev(W)
    note("bmm M=1024")
    yfull = host(B.bi_bmm(Ad, Wd))
    heads = [0, 5, 127]
    ref, s = oracle.bmm(A[heads][:, :64], W[heads])
    assert_within_tol(yfull[heads][:, :64], ref, s, "bmm heads rows 0..63")
    for M in (1, 16, 128):
        note(f"bmm M={M}")
        y = host(B.bi_bmm(Ad[:, :M].contiguous(), Wd))
        assert np.array_equal(y, yfull[:, :M]), f"M={M}"
        # strided head views (no copy) must agree too
        y2 = host(B.bi_bmm(Ad[:, :M], Wd))
        assert np.array_equal(y2, yfull[:, :M])
    g = inputs.rng(12345, 102)
    for trial in range(3):            # head subsets and row permutations
        hs = np.sort(g.choice(H, size=[1, 7, 33][trial], replace=False))
        rows = g.permutation(Mmax)[:[16, 129, 5][trial]]
        sub = Ad[torch.from_numpy(hs).cuda()][:, torch.from_numpy(rows).cuda()].contiguous()
        note(f"bmm subset trial {trial}")
        y = host(B.bi_bmm(sub, Wd[torch.from_numpy(hs).cuda()].contiguous()))
        assert np.array_equal(y, yfull[hs][:, rows])


def test_bmm_integer_exact_and_ragged():
    H, M, K, N = 6, 70, 136, 200
    A = inputs.randint_bf16((H, M, K), -3, 3, tag=(110,))
    W = inputs.randint_bf16((H, K, N), -3, 3, tag=(111,))
    ref, _ = oracle.bmm(A, W)
    note("bmm integer ragged")
    y = host(B.bi_bmm(dev(A), dev(W)))
    assert np.array_equal(y, rne_bf16_of_exact(ref))
    An = inputs.randn_bf16((H, M, K), tag=(112,))
    Wn = inputs.randn_bf16((H, K, N), tag=(113,))
    ref, s = oracle.bmm(An, Wn)
    y = host(B.bi_bmm(dev(An), dev(Wn)))
    assert_within_tol(y, ref, s, "bmm ragged gaussian")


# ----------------------------------------------------------------- NVFP4

def _nvfp4_weights(N, K, tag):
    x = inputs.rng(12345, *tag).standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    g = inputs.nvfp4_global_scale(x)
    W, Ws = inputs.nvfp4_quantize(x, g)
    return W, Ws, g


def test_nvfp4_integer_exact_pow2():
    M, N, K = 40, 200, 512
    W, Ws = inputs.random_nvfp4_pow2((N, K), tag=(120,))
    A = inputs.randint_bf16((M, K), -3, 3, tag=(121,))
    ref, _ = oracle.nvfp4_gemm(A, None, W, Ws, 1.0, K)
    note("nvfp4 integer pow2")
    y = host(B.bi_nvfp4_gemm(dev(A), dev(W), dev(Ws), 1.0))
    assert np.array_equal(y, rne_bf16_of_exact(ref))
    Aq, Aqs = inputs.random_nvfp4_pow2((M, K), tag=(122,))
    ref, _ = oracle.nvfp4_gemm(Aq, Aqs, W, Ws, 0.5, K)
    y = host(B.bi_nvfp4_gemm(dev(Aq), dev(W), dev(Ws), 0.5, A_scales=dev(Aqs)))
    assert np.array_equal(y, rne_bf16_of_exact(ref))


def _e2m1_e4m3_table():
    lut = np.array([oracle.e2m1_value(c) for c in range(16)])
    sv = np.array([oracle.e4m3_value(c) for c in range(256)])
    return lut, sv


@pytest.mark.parametrize("K,a_nvfp4", [(512, False), (480, False), (512, True)])
def test_nvfp4_decode_every_code_and_scale(K, a_nvfp4):
    """An identity A picks out single decoded weights: Y[k, n] = w(n, k)
    exactly (one nonzero product, exact in bf16).  Every one of the 16 codes
    appears under each of the 254 finite E4M3 scale bytes (0x7F and 0xFF are
    NaN).  K = 512 takes the raw-ring weight path, K = 480 (not a multiple of
    64) the register-staged one; with a_nvfp4 the identity is itself NVFP4
    (code 2 = 1.0 under scale 0x38 = 1.0), which decodes A as well."""
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    bpr = K // 16
    N = -(-finite.size // bpr)
    Ws = np.full(N * bpr, 0x38, np.uint8)
    Ws[:finite.size] = finite
    Ws = Ws.reshape(N, bpr)
    block = np.array([((2 * j + 1) << 4) | (2 * j) for j in range(8)], np.uint8)  # codes 0..15
    W = np.tile(block, N * bpr).reshape(N, K // 2)
    lut, sv = _e2m1_e4m3_table()
    # [K, N]; a zero weight sums to +0 (the fp32 accumulator starts at +0)
    want = lut[np.arange(K) % 16][:, None] * sv[Ws[:, np.arange(K) // 16]].T + 0.0
    want_bits = inputs.to_bf16_bits(want)
    assert np.array_equal(bf16_to_f64(want_bits), want)                          # exact in bf16
    if a_nvfp4:
        codes = np.zeros((K, K), np.uint8)
        codes[np.arange(K), np.arange(K)] = 2
        Aq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
        As = np.full((K, K // 16), 0x38, np.uint8)
        note(f"nvfp4 decode table K={K} (NVFP4 identity)")
        y = host(B.bi_nvfp4_gemm(dev(Aq), dev(W), dev(Ws), 1.0, A_scales=dev(As)))
    else:
        A = inputs.to_bf16_bits(np.eye(K))
        note(f"nvfp4 decode table K={K}")
        y = host(B.bi_nvfp4_gemm(dev(A), dev(W), dev(Ws), 1.0))
    assert np.array_equal(y, want_bits)


def test_nvfp4_equals_bf16_gemm_on_decoded_weights():
    """alpha == 1: bitwise the bf16 GEMM of the exactly decoded weights."""
    M, N, K = 96, 4096, 4096
    W, Ws, g = _nvfp4_weights(N, K, (123,))
    A = inputs.randn_bf16((M, K), tag=(124,))
    # decode with the oracle's decoders (test side), round (exactly) to bf16
    lut, sv = _e2m1_e4m3_table()
    q = np.empty((N, K), np.int64)
    q[:, 0::2] = W & 15
    q[:, 1::2] = W >> 4
    wdec = inputs.to_bf16_bits(lut[q] * np.repeat(sv[Ws], 16, axis=1))
    note("nvfp4 vs bf16 gemm")
    y4 = host(B.bi_nvfp4_gemm(dev(A), dev(W), dev(Ws), 1.0))
    yb = host(B.bi_gemm(dev(A), dev(wdec)))
    assert np.array_equal(y4, yb)


def test_nvfp4_activation_rows_quantised_alone():
    """W4A4: a row quantised alone with the batch's global scale gives the
    same codes, hence the same output row."""
    N, K, M = 2048, 4096, 64
    W, Ws, gw = _nvfp4_weights(N, K, (127,))
    x = inputs.rng(12345, 128).standard_normal((M, K)).astype(np.float32)
    ga = inputs.nvfp4_global_scale(x)
    Aq, Aqs = inputs.nvfp4_quantize(x, ga)
    alpha = float(np.float32(1.0) / (ga * gw))
    note("nvfp4 W4A4 full")
    yfull = host(B.bi_nvfp4_gemm(dev(Aq), dev(W), dev(Ws), alpha, A_scales=dev(Aqs)))
    ref, s = oracle.nvfp4_gemm(Aq, Aqs, W, Ws, alpha, K, rows=[0, 31, 63])
    assert_within_tol(yfull[[0, 31, 63]], ref, s, "w4a4 rows")
    for i in (0, 17, 63):
        qi, si = inputs.nvfp4_quantize(x[i:i + 1], ga)
        yi = host(B.bi_nvfp4_gemm(dev(qi), dev(W), dev(Ws), alpha, A_scales=dev(si)))
        assert np.array_equal(yi[0], yfull[i]), f"row {i}"


@pytest.mark.parametrize("N,K", [(1000, 1024), (24576, 4096), (300, 4608)])
def test_w4a4_streaming_small_m(N, K):
    """W4A4 at M <= 16 streams the weight with A decoded into LDS (at K =
    4608 the 16-row A no longer fits there, so M = 16 takes the tiled kernel
    while M <= 15 streams): every M in 1..16 is bitwise the forced tiled
    kernel and the M = 16 batch's prefix, also with A rows at a padded
    stride; power-of-two codes give the oracle's exact result; N(0,1) rows
    agree with the oracle within tolerance."""
    W, Ws, gw = _nvfp4_weights(N, K, (129, N))
    x = inputs.rng(12345, 130, N).standard_normal((16, K)).astype(np.float32)
    ga = inputs.nvfp4_global_scale(x)
    Aq, Aqs = inputs.nvfp4_quantize(x, ga)
    alpha = float(np.float32(1.0) / (ga * gw))
    Wd, Wsd = dev(W), dev(Ws)
    pad_q = np.zeros((16, K // 2 + 16), np.uint8)
    pad_s = np.zeros((16, K // 16 + 2), np.uint8)
    pad_q[:, :K // 2], pad_s[:, :K // 16] = Aq, Aqs
    Aqd, Aqsd = dev(Aq), dev(Aqs)
    Pq, Ps = dev(pad_q)[:, :K // 2], dev(pad_s)[:, :K // 16]
    note(f"w4a4 small M N={N} K={K} M=16")
    yfull = B.bi_nvfp4_gemm(Aqd, Wd, Wsd, alpha, A_scales=Aqsd)
    for M in range(1, 17):
        note(f"w4a4 small M N={N} K={K} M={M}")
        y = B.bi_nvfp4_gemm(Aqd[:M], Wd, Wsd, alpha, A_scales=Aqsd[:M])
        assert torch.equal(y, yfull[:M]), f"M={M} vs batch"
        assert torch.equal(y, B.bi_nvfp4_gemm(Aqd[:M], Wd, Wsd, alpha, A_scales=Aqsd[:M], tile_variant=13)), M
        assert torch.equal(y, B.bi_nvfp4_gemm(Pq[:M], Wd, Wsd, alpha, A_scales=Ps[:M])), f"M={M} padded"
    ref, s = oracle.nvfp4_gemm(Aq, Aqs, W, Ws, alpha, K, rows=[0, 7, 15])
    assert_within_tol(host(yfull)[[0, 7, 15]], ref, s, f"w4a4 N={N} K={K}")
    W2, Ws2 = inputs.random_nvfp4_pow2((N, K), tag=(131, N))
    A2, As2 = inputs.random_nvfp4_pow2((7, K), tag=(132, N))
    ref2, _ = oracle.nvfp4_gemm(A2, As2, W2, Ws2, 0.5, K)
    note(f"w4a4 small M integer-exact N={N} K={K}")
    y2 = host(B.bi_nvfp4_gemm(dev(A2), dev(W2), dev(Ws2), 0.5, A_scales=dev(As2)))
    assert np.array_equal(y2, rne_bf16_of_exact(ref2))


@pytest.mark.parametrize("N,K", [(24576, 4096), (6144, 4096), (8200, 2048), (1000, 4096)])
def test_w4a4_chunked_a_mid_m(N, K):
    """W4A4 at 16 < M <= 128 streams the weight with A's rows decoded into
    LDS chunk by chunk (two, four or eight row blocks; at least four
    wavefronts per workgroup, also when N gives fewer items than compute
    units): every M in {17, 20, 32, 33, 48, 63, 64, 65, 100, 127, 128} is
    bitwise the forced tiled kernel and the M = 128 batch's prefix, also with
    A rows at a padded stride, under wavefront caps {1, 7, #CU} and pipeline
    depths {1, 2, 4, 8}; N(0,1) rows agree with the oracle within tolerance;
    power-of-two codes give its exact result."""
    plan = B.plan_regimes(B.BI_OP_NVFP4_GEMM, N, K, 1)
    chunked = [r for r in plan if r["kind"] == "stream_a_chunks"]
    assert chunked and chunked[0]["m_min"] == 17 and chunked[-1]["m_max"] == 128, plan
    W, Ws, gw = _nvfp4_weights(N, K, (133, N))
    x = inputs.rng(12345, 134, N).standard_normal((128, K)).astype(np.float32)
    ga = inputs.nvfp4_global_scale(x)
    Aq, Aqs = inputs.nvfp4_quantize(x, ga)
    alpha = float(np.float32(1.0) / (ga * gw))
    Wd, Wsd = dev(W), dev(Ws)
    pad_q = np.zeros((128, K // 2 + 16), np.uint8)
    pad_s = np.zeros((128, K // 16 + 2), np.uint8)
    pad_q[:, :K // 2], pad_s[:, :K // 16] = Aq, Aqs
    Aqd, Aqsd = dev(Aq), dev(Aqs)
    Pq, Ps = dev(pad_q)[:, :K // 2], dev(pad_s)[:, :K // 16]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    note(f"w4a4 mid M N={N} K={K} M=128")
    yfull = B.bi_nvfp4_gemm(Aqd, Wd, Wsd, alpha, A_scales=Aqsd)
    for M in (17, 20, 32, 33, 48, 63, 64, 65, 100, 127, 128):
        note(f"w4a4 mid M N={N} K={K} M={M}")
        y = B.bi_nvfp4_gemm(Aqd[:M], Wd, Wsd, alpha, A_scales=Aqsd[:M])
        assert torch.equal(y, yfull[:M]), f"M={M} vs batch"
        assert torch.equal(y, B.bi_nvfp4_gemm(Aqd[:M], Wd, Wsd, alpha, A_scales=Aqsd[:M], tile_variant=13)), M
        assert torch.equal(y, B.bi_nvfp4_gemm(Pq[:M], Wd, Wsd, alpha, A_scales=Ps[:M])), f"M={M} padded"
        for mw in (1, 7, cus):
            assert torch.equal(y, B.bi_nvfp4_gemm(Aqd[:M], Wd, Wsd, alpha, A_scales=Aqsd[:M], max_workgroups=mw)), \
                (M, mw)
        for depth in (1, 2, 4, 8):
            assert torch.equal(y, B.bi_nvfp4_gemm(Aqd[:M], Wd, Wsd, alpha, A_scales=Aqsd[:M],
                                                  pipeline_depth=depth)), (M, depth)
    ref, s = oracle.nvfp4_gemm(Aq, Aqs, W, Ws, alpha, K, rows=[0, 17, 63, 127])
    assert_within_tol(host(yfull)[[0, 17, 63, 127]], ref, s, f"w4a4 mid M N={N} K={K}")
    W2, Ws2 = inputs.random_nvfp4_pow2((N, K), tag=(135, N))
    for mi in (40, 100):
        A2, As2 = inputs.random_nvfp4_pow2((mi, K), tag=(136, N, mi))
        rr = [0, mi // 2, mi - 1]
        ref2, _ = oracle.nvfp4_gemm(A2, As2, W2, Ws2, 0.5, K, rows=rr)
        note(f"w4a4 mid M integer-exact N={N} K={K} M={mi}")
        y2 = host(B.bi_nvfp4_gemm(dev(A2), dev(W2), dev(Ws2), 0.5, A_scales=dev(As2)))
        assert np.array_equal(y2[rr], rne_bf16_of_exact(ref2))


# ----------------------------------------------------------------- RMSNorm


@pytest.mark.parametrize("H,Mmax", [(512, 64), (4096, 2048), (1000, 33), (8, 5), (12288, 100)])
def test_rmsnorm_parity_and_invariance(H, Mmax):
    X = inputs.randn_bf16((Mmax, H), tag=(130, H))
    gam = inputs.uniform_bf16((H,), 0.5, 1.5, tag=(131, H))
    eps = 1e-6
    ref = oracle.rmsnorm(X, gam, eps)
    Xd, gd = dev(X), dev(gam)
    note(f"rmsnorm H={H} M={Mmax}")
    y = host(B.bi_rmsnorm(Xd, gd, eps))
    assert_within_tol(y, ref, np.abs(ref), f"rmsnorm H={H}")
    for M in sorted({1 << i for i in range(Mmax.bit_length()) if (1 << i) < Mmax} | {7, Mmax // 2}):
        yM = host(B.bi_rmsnorm(Xd[:M], gd, eps))
        assert np.array_equal(yM, y[:M])
    perm = inputs.rng(12345, 132).permutation(Mmax)
    yp = host(B.bi_rmsnorm(Xd[torch.from_numpy(perm).cuda()].contiguous(), gd, eps))
    assert np.array_equal(yp, y[perm])
    for mw in (1, 3, 1000):
        assert np.array_equal(host(B.bi_rmsnorm(Xd, gd, eps, max_workgroups=mw)), y)
    outs = {host(B.bi_rmsnorm(Xd, gd, eps)).tobytes() for _ in range(8)}
    assert len(outs) == 1


def test_rmsnorm_closed_forms_and_inplace():
    H = 4096
    gam = inputs.uniform_bf16((H,), 0.5, 1.5, tag=(133,))
    rows = np.stack([np.zeros(H), np.where(np.arange(H) % 5 == 0, -8.0, 8.0),
                     np.full(H, 0.25)])
    X = inputs.to_bf16_bits(rows)
    note("rmsnorm closed forms")
    y = host(B.bi_rmsnorm(dev(X), dev(gam), 1e-6))
    assert not bf16_to_f64(y[0]).any()
    gv = bf16_to_f64(gam)
    assert np.array_equal(bf16_to_f64(y[1]), np.sign(rows[1]) * gv)   # +-2^p row -> +-gamma
    assert np.array_equal(bf16_to_f64(y[2]), gv)                       # constant row, eps << ulp
    Xr = inputs.randn_bf16((64, H), tag=(134,))
    Xd = dev(Xr)
    ref = host(B.bi_rmsnorm(Xd, dev(gam), 1e-6))
    B.bi_rmsnorm(Xd, dev(gam), 1e-6, Xd)      # in place
    assert np.array_equal(host(Xd), ref)


def test_tile_shapes_bmm_and_nvfp4():
    """Every compiled tile shape gives the plan's bits for BMM and NVFP4."""
    nshapes = len(B.tile_shapes())
    A = inputs.randn_bf16((16, 100, 128), tag=(140,))
    W = inputs.randn_bf16((16, 128, 512), tag=(141,))
    Ad, Wd = dev(A), dev(W)
    y = host(B.bi_bmm(Ad, Wd))
    for v in range(1, nshapes + 1):
        note(f"bmm tile variant {v}")
        assert np.array_equal(host(B.bi_bmm(Ad, Wd, tile_variant=v)), y), v
    Wq, Ws, g = _nvfp4_weights(1000, 1024, (142,))
    X = inputs.randn_bf16((130, 1024), tag=(143,))
    Xd, Wqd, Wsd = dev(X), dev(Wq), dev(Ws)
    alpha = float(np.float32(1.0) / g)
    y = host(B.bi_nvfp4_gemm(Xd, Wqd, Wsd, alpha))
    for v in range(1, nshapes + 1):
        note(f"nvfp4 tile variant {v}")
        for rep in range(3):   # repeated: a timing-dependent LDS race shows as a rare mismatch
            assert np.array_equal(host(B.bi_nvfp4_gemm(Xd, Wqd, Wsd, alpha, tile_variant=v)), y), (v, rep)


@pytest.mark.parametrize("M,N,K", [(1000, 2600, 4160), (513, 1300, 2048), (2048, 6144, 4096), (77, 200, 64),
                                   (300, 256, 128), (260, 5000, 192)])
def test_nvfp4_pingpong_matches_classic_schedule(M, N, K):
    """The NVFP4 ping-pong kernel (256 x 256, tile variant 14) against the
    classic schedule of the same shape (13): ragged M and N, short K (one,
    two, three 64-column stages), several grid caps, each run repeated (a
    phase-ordering race would show as a rare mismatch); parity with the
    oracle on rows of the first and last M-tile."""
    Wq, Ws, g = _nvfp4_weights(N, K, (144, N))
    X = inputs.randn_bf16((M, K), tag=(145, M, N))
    Xd, Wqd, Wsd = dev(X), dev(Wq), dev(Ws)
    alpha = float(np.float32(1.0) / g)
    note(f"nvfp4 pingpong M={M} N={N} K={K} classic")
    y = host(B.bi_nvfp4_gemm(Xd, Wqd, Wsd, alpha, tile_variant=13))
    for mw in (0, 7, 64):
        for rep in range(2):
            note(f"nvfp4 pingpong M={M} N={N} K={K} grid cap {mw} rep {rep}")
            yp = host(B.bi_nvfp4_gemm(Xd, Wqd, Wsd, alpha, tile_variant=14, max_workgroups=mw))
            assert np.array_equal(yp, y), (M, N, K, mw, rep)
    rows = sorted({0, min(255, M - 1), M - 1})
    ref, s = oracle.nvfp4_gemm(X[rows], None, Wq, Ws, alpha, K)
    assert_within_tol(y[rows], ref, s, "nvfp4 pingpong")


def test_nvfp4_pingpong_decodes_every_code_and_scale():
    """The decode table of the ping-pong kernel: an identity A (bf16, 512
    rows) picks out single decoded weights, every one of the 16 codes under
    each of the 254 finite E4M3 scale bytes, through tile variant 14."""
    K = 512
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    bpr = K // 16
    N = -(-finite.size // bpr)
    Ws = np.full(N * bpr, 0x38, np.uint8)
    Ws[:finite.size] = finite
    Ws = Ws.reshape(N, bpr)
    block = np.array([((2 * j + 1) << 4) | (2 * j) for j in range(8)], np.uint8)
    W = np.tile(block, N * bpr).reshape(N, K // 2)
    lut, sv = _e2m1_e4m3_table()
    want = lut[np.arange(K) % 16][:, None] * sv[Ws[:, np.arange(K) // 16]].T + 0.0
    want_bits = inputs.to_bf16_bits(want)
    A = inputs.to_bf16_bits(np.eye(K))
    note("nvfp4 pingpong decode table")
    y = host(B.bi_nvfp4_gemm(dev(A), dev(W), dev(Ws), 1.0, tile_variant=14))
    assert np.array_equal(y, want_bits)


@pytest.mark.parametrize("H,M,K,N", [(5, 70, 64, 200), (3, 33, 128, 512), (2, 129, 256, 136),
                                     (128, 1, 128, 512), (7, 1000, 128, 264)])
def test_bmm_short_k_kernel(H, M, K, N):
    """The streaming BMM kernel (K in {64, 128, 256}): integer inputs give
    bf16_rne(exact) bit for bit, Gaussian inputs stay within the oracle's
    tolerance, and the bits equal those of every tiled variant (the same
    per-element MFMA chain), whatever the heads, rows and grid."""
    Ai = inputs.randint_bf16((H, M, K), -3, 3, tag=(150, K))
    Wi = inputs.randint_bf16((H, K, N), -3, 3, tag=(151, K))
    ref, _ = oracle.bmm(Ai, Wi)
    note(f"bmm short-K integer H={H} M={M} K={K} N={N}")
    assert np.array_equal(host(B.bi_bmm(dev(Ai), dev(Wi))), rne_bf16_of_exact(ref))
    A = inputs.randn_bf16((H, M, K), tag=(152, K))
    W = inputs.randn_bf16((H, K, N), tag=(153, K))
    Ad, Wd = dev(A), dev(W)
    note(f"bmm short-K gaussian H={H} M={M} K={K} N={N}")
    y = host(B.bi_bmm(Ad, Wd))
    hs = sorted({0, H - 1})
    ref, s = oracle.bmm(A[hs][:, :min(M, 64)], W[hs])
    assert_within_tol(y[hs][:, :min(M, 64)], ref, s, "bmm short-K")
    for v in (2, 3, 10):        # 256x128, 128x128, 128x128 (4x2 waves) tiled kernels
        note(f"bmm short-K vs tile variant {v}")
        assert np.array_equal(host(B.bi_bmm(Ad, Wd, tile_variant=v)), y), v
    for mw in (1, 3, 8, 1000):
        assert np.array_equal(host(B.bi_bmm(Ad, Wd, max_workgroups=mw)), y), mw
    if M > 1:
        assert np.array_equal(host(B.bi_bmm(Ad[:, :1].contiguous(), Wd)), y[:, :1])
        rows = inputs.rng(12345, 154).permutation(M)[:max(1, M // 3)]
        r = torch.from_numpy(rows).cuda()
        assert np.array_equal(host(B.bi_bmm(Ad[:, r].contiguous(), Wd)), y[:, rows])
    if H > 1:
        assert np.array_equal(host(B.bi_bmm(Ad[H - 1:], Wd[H - 1:])), y[H - 1:])
    outs = {host(B.bi_bmm(Ad, Wd)).tobytes() for _ in range(4)}
    assert len(outs) == 1
