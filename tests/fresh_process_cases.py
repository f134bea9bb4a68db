"""Seeded cases whose output digests must be the same in every process.

Imported by the GPU test of run-to-run determinism across processes, and run
as a child process by that test (``python tests/fresh_process_cases.py``
prints one JSON line of digests).  Each case is a small but multi-tile call
of one entry point on inputs from the seeded generators.
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def digests() -> dict:
    import numpy as np
    import torch

    from invariant_deterministic_bi_amd import binding as B
    from invariant_deterministic_bi_amd import inputs

    def d(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    def h(t):
        torch.cuda.synchronize()
        return hashlib.sha256(t.contiguous().view(torch.uint8).cpu().numpy().tobytes()).hexdigest()

    out = {}
    A = d(inputs.randn_bf16((300, 4096), tag=(800,)))
    W = d(inputs.randn_bf16((6144, 4096), 0.02, tag=(801,)))
    out["gemm_qkv_M300"] = h(B.bi_gemm(A, W))
    out["gemm_qkv_M5"] = h(B.bi_gemm(A[:5], W))
    x = inputs.rng(12345, 802).standard_normal((4096, 4096)).astype(np.float32) * np.float32(0.02)
    g = inputs.nvfp4_global_scale(x)
    Wq, Ws = inputs.nvfp4_quantize(x, g)
    alpha = float(np.float32(1.0) / g)
    out["nvfp4_M300"] = h(B.bi_nvfp4_gemm(A, d(Wq), d(Ws), alpha))
    out["nvfp4_M3"] = h(B.bi_nvfp4_gemm(A[:3], d(Wq), d(Ws), alpha))
    gam = d(inputs.uniform_bf16((4096,), 0.5, 1.5, tag=(803,)))
    out["rmsnorm_M300"] = h(B.bi_rmsnorm(A, gam, 1e-6))
    Ab = d(inputs.randn_bf16((16, 64, 128), tag=(804,)))
    Wb = d(inputs.randn_bf16((16, 128, 512), tag=(805,)))
    out["bmm_16x64"] = h(B.bi_bmm(Ab, Wb))
    q = d(inputs.randn_bf16((3, 16, 576), tag=(806,)))
    kv = d(inputs.randn_bf16((3, 1500, 576), tag=(807,)))
    lens = torch.tensor([1500, 3, 1025], dtype=torch.int32, device="cuda")
    out["mla_decode_3req"] = h(B.bi_mla_decode(q, kv, lens, 0.072, 512))
    return out


if __name__ == "__main__":
    print(json.dumps(digests(), sort_keys=True), flush=True)
