"""GPU tests of bi_mla_decode_noalloc, the decode-attention entry point for
callers that cannot allocate: its chunk partials live in a scratch array the
library holds on each GPU.  Its outputs must be bitwise those of
bi_mla_decode (with and without a caller workspace) on two calls in a row,
the second smaller than the first, and it must allocate nothing."""
import math

import numpy as np
import pytest
import torch

from invariant_deterministic_bi_amd import inputs
from invariant_deterministic_bi_amd import binding as B
from gpu_util import dev, note

pytestmark = pytest.mark.gpu


def _case(Bn, H, Lmax, Dqk, lo, tag):
    lens = inputs.rng(12345, 600, tag).integers(lo, Lmax + 1, Bn).astype(np.int32)
    q = dev(inputs.randn_bf16((Bn, H, Dqk), 1.0, tag=(601, tag)))
    kv = dev(inputs.randn_bf16((Bn, Lmax, Dqk), 1.0, tag=(602, tag)))
    return q, kv, torch.from_numpy(lens).cuda()


def test_noalloc_matches_bi_mla_decode_twice():
    """Call 1: 64 requests of 1024..4096 tokens, 16 heads, Dqk 576, Dv 512
    (64 head groups < #CU, so the chunked schedule runs on the scratch
    array).  Call 2: 8 requests of 1..2048 tokens.  Both bitwise equal to
    bi_mla_decode with a caller workspace and without one; the device's free
    memory is unchanged by a call."""
    scale = 1.0 / math.sqrt(192.0)
    Dv = 512
    for (Bn, H, Lmax, lo, tag) in ((64, 16, 4096, 1024, 1), (8, 16, 2048, 1, 2)):
        q, kv, lens = _case(Bn, H, Lmax, 576, lo, tag)
        need = B.mla_decode_workspace_size(Bn, H, Lmax, 576, Dv)
        assert 0 < need <= B.MLA_SCRATCH_BYTES
        out = torch.empty((Bn, H, Dv), dtype=torch.bfloat16, device="cuda")
        note(f"noalloc B={Bn} Lmax={Lmax} first call")
        B.bi_mla_decode_noalloc(q, kv, lens, scale, Dv, out)
        out.zero_()
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]   # after every kernel module this loop uses is loaded
        note(f"noalloc B={Bn} Lmax={Lmax} second call")
        B.bi_mla_decode_noalloc(q, kv, lens, scale, Dv, out)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ref_ws = B.bi_mla_decode(q, kv, lens, scale, Dv, workspace=ws)
        ref = B.bi_mla_decode(q, kv, lens, scale, Dv)
        assert torch.equal(out, ref_ws), (Bn, Lmax)
        assert torch.equal(out, ref), (Bn, Lmax)


def test_noalloc_other_shapes_and_limit():
    """A shape the fp32 kernel serves (no scratch needed) and a small
    matrix-core shape give bi_mla_decode's bits; a call whose chunked
    schedule would need more than the scratch array is refused with
    BI_ERR_UNSUPPORTED before any launch."""
    scale = 0.125
    for (Bn, H, Lmax, Dqk, Dv, tag) in ((5, 4, 300, 256, 256, 3), (3, 20, 2500, 128, 64, 4)):
        q, kv, lens = _case(Bn, H, Lmax, Dqk, 0, tag)
        out = torch.empty((Bn, H, Dv), dtype=torch.bfloat16, device="cuda")
        note(f"noalloc Dqk={Dqk} Dv={Dv}")
        B.bi_mla_decode_noalloc(q, kv, lens, scale, Dv, out)
        assert torch.equal(out, B.bi_mla_decode(q, kv, lens, scale, Dv, workspace=True))
    Bn, H, Lmax = 100, 16, 16384
    assert B.mla_decode_workspace_size(Bn, H, Lmax, 576, 512) > B.MLA_SCRATCH_BYTES
    q = torch.empty((Bn, H, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((Bn, Lmax, 576), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((Bn,), Lmax, dtype=torch.int32, device="cuda")
    out = torch.empty((Bn, H, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.BiError) as e:
        B.bi_mla_decode_noalloc(q, kv, lens, scale, 512, out)
    assert e.value.status == B.BI_ERR_UNSUPPORTED
