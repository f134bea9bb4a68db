"""GPU parity and invariance tests of bi_mla_decode, decode attention over a
latent KV cache: each (request, head) output must match the fp64 oracle
within the derived bound, and be bitwise the same alone, in any batch, with
any head subset, grid cap or cache capacity."""
import math

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_bi_amd import inputs
from invariant_deterministic_bi_amd import binding as B
from harness import assert_within_tol, mla_rel_bound, rne_bf16_of_exact, bf16_to_f64
from gpu_util import dev, host, note

pytestmark = pytest.mark.gpu


def lens_dev(lens):
    return torch.tensor(np.asarray(lens, np.int32), dtype=torch.int32, device="cuda")


def check_parity(o_bits, q, kv, lens, scale, Dv, what):
    ref, s = oracle.mla_decode(q, kv, lens, scale, Dv)
    c = mla_rel_bound(q, kv, lens, scale)
    # assert_within_tol adds 1e-3*S; the extra term lifts the bound to c*S
    assert_within_tol(o_bits, ref, s, what, extra=(c - 1e-3) * s)


@pytest.mark.parametrize("lens,H,Dqk,Dv,Lmax", [([1, 37, 300, 0, 1029], 16, 576, 512, 1100),
                                                ([4096, 2500], 16, 576, 512, 4096),
                                                ([7, 64, 255, 256, 257], 3, 64, 64, 260),
                                                ([5, 0, 13], 2, 8, 8, 16),
                                                ([200, 33], 4, 1024, 1024, 200),
                                                ([100, 7, 64], 20, 576, 512, 128),
                                                ([33, 1], 5, 128, 64, 40),
                                                # matrix-core kernel with a partial last K chunk and value block
                                                ([50, 1100, 0], 16, 568, 392, 1200),
                                                ([9, 70], 3, 40, 24, 80)])
def test_mla_decode_parity_and_requests_alone(lens, H, Dqk, Dv, Lmax):
    Bn = len(lens)
    scale = 1.0 / math.sqrt(192.0)
    q = inputs.randn_bf16((Bn, H, Dqk), 1.0, tag=(500, Dqk, Lmax))
    kv = inputs.randn_bf16((Bn, Lmax, Dqk), 1.0, tag=(501, Dqk, Lmax))
    qd, kvd = dev(q), dev(kv)
    note(f"mla_decode lens={lens} H={H} Dqk={Dqk} Dv={Dv} Lmax={Lmax}")
    o = host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv))
    check_parity(o, q, kv, lens, scale, Dv, "mla_decode")
    # one workgroup per 1024-token chunk plus the fold: the same bits
    assert np.array_equal(host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv, workspace=True)), o)
    for b in range(Bn):
        if lens[b] == 0:
            assert not o[b].any(), b
        # the request alone, with only its own cache rows
        Lb = max(lens[b], 1)
        alone = host(B.bi_mla_decode(qd[b:b + 1].contiguous(), kvd[b:b + 1, :Lb].contiguous(),
                                     lens_dev([lens[b]]), scale, Dv))
        assert np.array_equal(alone[0], o[b]), b
    # one head alone
    h = H - 1
    one = host(B.bi_mla_decode(qd[:, h:h + 1].contiguous(), kvd, lens_dev(lens), scale, Dv))
    assert np.array_equal(one[:, 0], o[:, h])
    for mw in (1, 7):
        assert np.array_equal(host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv, max_workgroups=mw)), o)
    outs = {host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv)).tobytes() for _ in range(3)}
    assert len(outs) == 1


def test_mla_decode_chunk_boundaries_and_schedules():
    """Requests ending on, just before and just after the 1024-token chunk
    boundaries and the 32-token block boundaries: parity; the chunked
    schedule (workspace, first chunks first), the one-workgroup schedule
    (its copy stream running across the chunks), both under grid caps that
    make a workgroup take several units, and the no-allocation entry point
    all give the same bits."""
    lens = [1024, 1025, 2047, 2048, 2049, 3072, 32, 31, 0, 1]
    Bn, H, Dqk, Dv, Lmax = len(lens), 16, 576, 512, 3100
    scale = 1.0 / math.sqrt(192.0)
    q = inputs.randn_bf16((Bn, H, Dqk), 1.0, tag=(505, Lmax))
    kv = inputs.randn_bf16((Bn, Lmax, Dqk), 1.0, tag=(506, Lmax))
    qd, kvd = dev(q), dev(kv)
    note("mla_decode chunk boundaries and schedules")
    o = host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv))
    pick = [0, 1, 3, 4, 6, 7]
    check_parity(o[pick], q[pick], kv[pick], [lens[i] for i in pick], scale, Dv, "mla_decode chunk boundaries")
    assert not o[8].any()
    ws = torch.empty(B.mla_decode_workspace_size(Bn, H, Lmax, Dqk, Dv), dtype=torch.uint8, device="cuda")
    assert np.array_equal(host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv, workspace=ws)), o)
    for mw in (1, 3, 100):
        assert np.array_equal(host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv, workspace=ws,
                                                   max_workgroups=mw)), o), mw
    for mw in (2, 5):
        assert np.array_equal(host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv, max_workgroups=mw)), o), mw
    on = torch.empty((Bn, H, Dv), dtype=torch.bfloat16, device="cuda")
    B.bi_mla_decode_noalloc(qd, kvd, lens_dev(lens), scale, Dv, on)
    assert np.array_equal(host(on), o)


def test_mla_decode_batch_composition_and_capacity():
    """A request's output is the same bits inside batches of other requests of
    other lengths, and whether the dense cache layout holds 4096 or 5000 rows
    per request (matrix-core kernel, Dqk 576 / Dv 512)."""
    H, Dqk, Dv = 16, 576, 512
    scale = 0.0721
    q = inputs.randn_bf16((6, H, Dqk), 1.0, tag=(510,))
    kv = inputs.randn_bf16((6, 4096, Dqk), 1.0, tag=(511,))
    lens = [3000, 1, 4096, 517, 0, 2048]
    qd, kvd = dev(q), dev(kv)
    note("mla_decode batch composition")
    full = host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv))
    # sub-batches in another order
    idx = [5, 2, 0]
    sub = host(B.bi_mla_decode(qd[idx].contiguous(), kvd[idx].contiguous(), lens_dev([lens[i] for i in idx]),
                               scale, Dv))
    for j, i in enumerate(idx):
        assert np.array_equal(sub[j], full[i]), i
    # the same requests in a 5000-row layout
    big = torch.zeros((6, 5000, Dqk), dtype=torch.bfloat16, device="cuda")
    big[:, :4096] = kvd
    wide = host(B.bi_mla_decode(qd, big, lens_dev(lens), scale, Dv))
    assert np.array_equal(wide, full)
    # sampled parity of the whole batch
    check_parity(full[[0, 2, 5]], q[[0, 2, 5]], kv[[0, 2, 5]], [lens[i] for i in (0, 2, 5)], scale, Dv,
                 "mla_decode batch")


def test_mla_decode_long_request():
    """The 16384-token capacity: one request of 16384 tokens, parity."""
    H, Dqk, Dv, L = 4, 576, 512, 16384
    scale = 1.0 / math.sqrt(192.0)
    q = inputs.randn_bf16((1, H, Dqk), 1.0, tag=(520,))
    kv = inputs.randn_bf16((1, L, Dqk), 1.0, tag=(521,))
    note("mla_decode L=16384")
    o = host(B.bi_mla_decode(dev(q), dev(kv), lens_dev([L]), scale, Dv))
    check_parity(o, q, kv, [L], scale, Dv, "mla_decode long")
    ow = host(B.bi_mla_decode(dev(q), dev(kv), lens_dev([L]), scale, Dv, workspace=True))
    assert np.array_equal(ow, o)


def test_mla_decode_exact_cases():
    """scale 0 makes every weight exactly 1: the output is the exact mean of
    the value rows, bf16-rounded once (integer values, L a power of two).  A
    one-token request returns its value row exactly."""
    H, Dqk, Dv = 4, 128, 64
    q = inputs.randn_bf16((3, H, Dqk), 1.0, tag=(530,))
    kv = inputs.randint_bf16((3, 1024, Dqk), -3, 3, tag=(531,))
    lens = [1024, 1, 256]
    note("mla_decode exact cases")
    o = host(B.bi_mla_decode(dev(q), dev(kv), lens_dev(lens), 0.0, Dv))
    v = bf16_to_f64(kv)
    for b, L in enumerate(lens):
        mean = v[b, :L, :Dv].sum(axis=0) / L
        exp = rne_bf16_of_exact(np.broadcast_to(mean, (H, Dv)))
        assert np.array_equal(o[b], exp), b
    # a one-token request with a nonzero scale still returns v_0 exactly
    o1 = host(B.bi_mla_decode(dev(q), dev(kv), lens_dev([1, 1, 1]), 0.37, Dv))
    for b in range(3):
        assert np.array_equal(o1[b], np.broadcast_to(kv[b, 0, :Dv], (H, Dv))), b


def test_mla_decode_lens_clamped_and_empty():
    """lens outside [0, Lmax] are clamped by the kernel; B == 0 is a no-op."""
    H, Dqk, Dv, Lmax = 2, 64, 32, 40
    q = inputs.randn_bf16((3, H, Dqk), 1.0, tag=(540,))
    kv = inputs.randn_bf16((3, Lmax, Dqk), 1.0, tag=(541,))
    qd, kvd = dev(q), dev(kv)
    note("mla_decode clamped lens")
    o = host(B.bi_mla_decode(qd, kvd, lens_dev([-5, 1000, 17]), 0.125, Dv))
    ref = host(B.bi_mla_decode(qd, kvd, lens_dev([0, Lmax, 17]), 0.125, Dv))
    assert np.array_equal(o, ref)
    assert not o[0].any()
    e = B.bi_mla_decode(qd[:0], kvd[:0], lens_dev([]), 0.125, Dv)
    assert e.shape == (0, H, Dv)


def test_mla_decode_bench_configuration_sampled():
    """The timed workload's launch configuration: 64 requests of 1024..4096
    tokens (the same seeded lengths), 16 heads, Dqk 576, Dv 512, Lmax 4096.
    Sampled requests are checked against the oracle, and each alone is
    bitwise its row of the batch."""
    Bn, H, Dqk, Dv, Lmax = 64, 16, 576, 512, 4096
    lens = inputs.rng(12345, 21).integers(1024, Lmax + 1, Bn).astype(np.int32)
    scale = 1.0 / 192 ** 0.5
    q = inputs.randn_bf16((Bn, H, Dqk), 1.0, tag=(550,))
    kv = inputs.randn_bf16((Bn, Lmax, Dqk), 1.0, tag=(551,))
    qd, kvd = dev(q), dev(kv)
    note("mla_decode bench configuration B=64 H=16 Lmax=4096")
    o = host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv))
    pick = [0, int(np.argmax(lens)), int(np.argmin(lens)), Bn - 1]
    check_parity(o[pick], q[pick], kv[pick], lens[pick], scale, Dv, "mla_decode bench config")
    ws = torch.empty(B.mla_decode_workspace_size(Bn, H, Lmax, Dqk, Dv), dtype=torch.uint8, device="cuda")
    assert np.array_equal(host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv, workspace=ws)), o)
    for mw in (1, 37):
        assert np.array_equal(host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv, workspace=ws,
                                                   max_workgroups=mw)), o)
    for b in pick:
        alone = host(B.bi_mla_decode(qd[b:b + 1].contiguous(), kvd[b:b + 1].contiguous(), lens_dev(lens[b:b + 1]),
                                     scale, Dv))
        assert np.array_equal(alone[0], o[b]), b
        alone = host(B.bi_mla_decode(qd[b:b + 1].contiguous(), kvd[b:b + 1].contiguous(), lens_dev(lens[b:b + 1]),
                                     scale, Dv, workspace=True))
        assert np.array_equal(alone[0], o[b]), b


def test_mla_decode_moving_max():
    """Scores that rise (or fall) along the sequence make the running max
    change in every 32-token block and every chunk, so every rescale and
    every chunk fold is exercised; parity, and the same bits with and
    without the workspace."""
    H, Dqk, Dv, L = 16, 576, 512, 3000
    q = inputs.randn_bf16((2, H, Dqk), 0.5, tag=(560,))
    kv = inputs.randn_bf16((2, L, Dqk), 0.5, tag=(561,))
    ramp = np.linspace(-6.0, 6.0, L)
    q[:, :, Dqk - 1] = inputs.to_bf16_bits(np.full((2, H), 4.0))
    kv[0, :, Dqk - 1] = inputs.to_bf16_bits(ramp)          # rising scores
    kv[1, :, Dqk - 1] = inputs.to_bf16_bits(ramp[::-1])    # falling scores
    scale = 1.0 / math.sqrt(192.0)
    qd, kvd = dev(q), dev(kv)
    note("mla_decode moving max")
    o = host(B.bi_mla_decode(qd, kvd, lens_dev([L, L]), scale, Dv))
    check_parity(o, q, kv, [L, L], scale, Dv, "mla_decode moving max")
    assert np.array_equal(host(B.bi_mla_decode(qd, kvd, lens_dev([L, L]), scale, Dv, workspace=True)), o)


def test_absorbed_mla_decode_pipeline_request_alone():
    """The absorbed MLA decode step end to end, three library calls: the
    query's no-rope part times W_UK per head (bi_bmm, [H, B, 128] x [H, 128,
    512]), joined with its rope part into the 576-wide latent query; attention
    over the latent cache (bi_mla_decode, with and without the workspace);
    the latent output times W_UV per head (bi_bmm, [H, B, 512] x [H, 512,
    128]).  Each request run alone gives bitwise its rows of the batch."""
    Bn, H, L = 8, 16, 2500
    lens = inputs.rng(12345, 570).integers(1, L + 1, Bn).astype(np.int32)
    q_nope = dev(inputs.randn_bf16((Bn, H, 128), 1.0, tag=(571,)))
    q_pe = dev(inputs.randn_bf16((Bn, H, 64), 1.0, tag=(572,)))
    w_uk = dev(inputs.randn_bf16((H, 128, 512), 0.09, tag=(573,)))
    w_uv = dev(inputs.randn_bf16((H, 512, 128), 0.05, tag=(574,)))
    kv = dev(inputs.randn_bf16((Bn, L, 576), 1.0, tag=(575,)))
    scale = 1.0 / math.sqrt(192.0)

    def step(rows, workspace):
        qn = q_nope[rows].permute(1, 0, 2).contiguous()                      # [H, b, 128]
        q_lat = B.bi_bmm(qn, w_uk).permute(1, 0, 2)                          # [b, H, 512] view
        q = torch.cat([q_lat, q_pe[rows]], dim=2).contiguous()               # [b, H, 576]
        o_lat = B.bi_mla_decode(q, kv[rows].contiguous(), lens_dev(lens[rows]), scale, 512,
                                workspace=workspace)
        return B.bi_bmm(o_lat.permute(1, 0, 2).contiguous(), w_uv)           # [H, b, 128]

    note("absorbed MLA decode pipeline")
    allr = list(range(Bn))
    full = host(step(allr, None))
    assert np.array_equal(host(step(allr, True)), full)
    for b in (0, 3, Bn - 1):
        alone = host(step([b], None))
        assert np.array_equal(alone[:, 0], full[:, b]), b
    sub = [6, 1, 4]
    part = host(step(sub, True))
    for j, b in enumerate(sub):
        assert np.array_equal(part[:, j], full[:, b]), b


@pytest.mark.parametrize("Dqk,Dv", [(256, 256), (1024, 1024)])
def test_mla_decode_fp32_kernel_large_capacity(Dqk, Dv):
    """Shapes the fp32 (VALU) kernel serves, at its larger LDS capacity
    (Lmax above 4096 keeps up to 16384 weights per workgroup): parity; each
    request alone; the requests of at most 4096 tokens bitwise the same in a
    4096-row layout (the smaller capacity) as in the 5000-row one; and one
    request of 16384 tokens."""
    H, Lmax = 4, 5000
    lens = [5000, 4096, 1, 0, 3000]
    Bn = len(lens)
    scale = 1.0 / math.sqrt(192.0)
    q = inputs.randn_bf16((Bn, H, Dqk), 1.0, tag=(580, Dqk))
    kv = inputs.randn_bf16((Bn, Lmax, Dqk), 1.0, tag=(581, Dqk))
    qd, kvd = dev(q), dev(kv)
    note(f"mla_decode fp32 kernel Dqk={Dqk} Lmax={Lmax}")
    o = host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv))
    check_parity(o, q, kv, lens, scale, Dv, "mla_decode fp32 kernel Lmax 5000")
    assert np.array_equal(host(B.bi_mla_decode(qd, kvd, lens_dev(lens), scale, Dv, workspace=True)), o)
    for b in range(Bn):
        alone = host(B.bi_mla_decode(qd[b:b + 1].contiguous(), kvd[b:b + 1].contiguous(), lens_dev([lens[b]]),
                                     scale, Dv))
        assert np.array_equal(alone[0], o[b]), b
    small = [1, 2, 3, 4]
    narrow = host(B.bi_mla_decode(qd[small].contiguous(), kvd[small, :4096].contiguous(),
                                  lens_dev([lens[i] for i in small]), scale, Dv))
    assert np.array_equal(narrow, o[small])
    L = 16384
    q1 = inputs.randn_bf16((1, H, Dqk), 1.0, tag=(582, Dqk))
    kv1 = inputs.randn_bf16((1, L, Dqk), 1.0, tag=(583, Dqk))
    note(f"mla_decode fp32 kernel Dqk={Dqk} L={L}")
    o1 = host(B.bi_mla_decode(dev(q1), dev(kv1), lens_dev([L]), scale, Dv))
    check_parity(o1, q1, kv1, [L], scale, Dv, "mla_decode fp32 kernel L 16384")
