"""GPU checks of the fixed-plan launch option: with fixed_plan the tiled
kernel runs one tile shape per (operation, operand formats, N, K) at every M,
so no kernel or tile is chosen from M; its rows must be bitwise those of the
default dispatch (which also chooses by M) and of its own full batch."""
import numpy as np
import pytest
import torch

from invariant_deterministic_bi_amd import inputs
from invariant_deterministic_bi_amd import binding as B
from gpu_util import dev, note

pytestmark = pytest.mark.gpu

# the M of every regime the default dispatch uses at these shapes: streaming
# (M <= 16), register streaming or chunked A (to 128), each tile band, and
# the many-rows plan itself
MS = (1, 2, 9, 16, 17, 64, 65, 128, 129, 256, 700, 1300, 2048)


@pytest.mark.parametrize("N,K", [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288), (256, 512)])
def test_fixed_plan_bf16_same_bits(N, K):
    A = dev(inputs.randn_bf16((2048, K), 1.0, tag=(700, N, K)))
    W = dev(inputs.randn_bf16((N, K), 0.02, tag=(701, N, K)))
    note(f"fixed plan bf16 N={N} K={K} M=2048")
    full = B.bi_gemm(A, W, fixed_plan=True)
    assert torch.equal(full, B.bi_gemm(A, W)), "full batch: fixed plan vs default"
    for M in MS:
        note(f"fixed plan bf16 N={N} K={K} M={M}")
        y = B.bi_gemm(A[:M], W, fixed_plan=True)
        assert torch.equal(y, full[:M]), f"M={M}: fixed plan vs its full batch"
        assert torch.equal(y, B.bi_gemm(A[:M], W)), f"M={M}: fixed plan vs default"


def test_fixed_plan_nvfp4_same_bits():
    N, K = 24576, 4096
    w = inputs.rng(12345, 702).standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    gw = inputs.nvfp4_global_scale(w)
    Wq, Ws = inputs.nvfp4_quantize(w, gw)
    Wd, Wsd = dev(Wq), dev(Ws)
    x = inputs.rng(12345, 703).standard_normal((2048, K)).astype(np.float32)
    A = dev(inputs.randn_bf16((2048, K), 1.0, tag=(704,)))
    alpha = float(np.float32(1.0) / gw)
    note("fixed plan nvfp4 bf16 A M=2048")
    full = B.bi_nvfp4_gemm(A, Wd, Wsd, alpha, fixed_plan=True)
    for M in (1, 16, 17, 64, 65, 128, 129, 700, 2048):
        note(f"fixed plan nvfp4 bf16 A M={M}")
        y = B.bi_nvfp4_gemm(A[:M], Wd, Wsd, alpha, fixed_plan=True)
        assert torch.equal(y, full[:M]), M
        assert torch.equal(y, B.bi_nvfp4_gemm(A[:M], Wd, Wsd, alpha)), M
    # NVFP4 A, quantised with the batch's global scale
    ga = inputs.nvfp4_global_scale(x)
    Aq, Aqs = inputs.nvfp4_quantize(x, ga)
    Aqd, Aqsd = dev(Aq), dev(Aqs)
    alpha4 = float(np.float32(1.0) / (np.float32(ga) * np.float32(gw)))
    note("fixed plan nvfp4 NVFP4 A M=2048")
    full4 = B.bi_nvfp4_gemm(Aqd, Wd, Wsd, alpha4, A_scales=Aqsd, fixed_plan=True)
    for M in (1, 16, 17, 128, 129, 2048):
        note(f"fixed plan nvfp4 NVFP4 A M={M}")
        y = B.bi_nvfp4_gemm(Aqd[:M], Wd, Wsd, alpha4, A_scales=Aqsd[:M], fixed_plan=True)
        assert torch.equal(y, full4[:M]), M
        assert torch.equal(y, B.bi_nvfp4_gemm(Aqd[:M], Wd, Wsd, alpha4, A_scales=Aqsd[:M])), M


def test_fixed_plan_grouped_same_bits():
    E, N, K = 8, 4096, 1024
    sizes = [3, 0, 40, 150, 1, 300, 17, 700]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    T = int(off[-1])
    A = dev(inputs.randn_bf16((T, K), 1.0, tag=(705,)))
    W = dev(inputs.randn_bf16((E, N, K), 0.02, tag=(706,)))
    offs = torch.tensor(off, dtype=torch.int64, device="cuda")
    note(f"fixed plan grouped E={E} N={N} K={K} T={T}")
    y = B.bi_grouped_gemm(A, W, offs, fixed_plan=True)
    assert torch.equal(y, B.bi_grouped_gemm(A, W, offs))
    for e in (0, 3, 7):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            assert torch.equal(y[r0:r1], B.bi_gemm(A[r0:r1], W[e], fixed_plan=True)), e
