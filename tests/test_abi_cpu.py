"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, plans are keyed on (op, N, K) only, and argument validation
rejects bad calls before anything is launched.

Every call below is rejected by validation or is an M == 0 no-op, so no
kernel is ever launched (fake addresses are never dereferenced).
"""
import ctypes
import os
import re

import pytest

from invariant_deterministic_bi_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "bi.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    lib = B.lib()
    names = header_functions()
    assert {"bi_gemm", "bi_bmm", "bi_nvfp4_gemm", "bi_rmsnorm", "bi_plan_query",
            "bi_status_str"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libbi.so does not export {n}"


def test_status_strings():
    for s in range(8):
        assert B.status_str(s)
    assert "VALUE" in B.status_str(B.BI_ERR_VALUE)
    assert "UNSUPPORTED" in B.status_str(B.BI_ERR_UNSUPPORTED)
    assert B.version().startswith("bi ")


@pytest.mark.parametrize("N,K", [(256, 512), (6144, 4096), (4096, 4096), (24576, 4096),
                                 (4096, 12288), (200, 544)])
def test_plan_is_fixed_per_NK(N, K):
    p = B.plan_query(B.BI_OP_GEMM, N, K)
    assert p["mfma_m"] == 16 and p["mfma_n"] == 16 and p["mfma_k"] == 32
    assert p["bm"] > 0 and p["bn"] > 0 and p["bk"] == 64
    # the same key always gives the same plan
    assert p == B.plan_query(B.BI_OP_GEMM, N, K)


def test_nvfp4_plan_uses_the_bf16_recipe():
    # same MFMA instruction and K order as the bf16 GEMM for the same (N, K)
    g = B.plan_query(B.BI_OP_GEMM, 24576, 4096)
    f = B.plan_query(B.BI_OP_NVFP4_GEMM, 24576, 4096)
    for k in ("mfma_m", "mfma_n", "mfma_k", "bk"):
        assert g[k] == f[k]


def test_plan_query_rejects():
    with pytest.raises(B.BiError) as e:
        B.plan_query(B.BI_OP_GEMM, 256, 12)
    assert e.value.status == B.BI_ERR_SHAPE
    with pytest.raises(B.BiError) as e:
        B.plan_query(B.BI_OP_NVFP4_GEMM, 256, 48)
    assert e.value.status == B.BI_ERR_SHAPE
    with pytest.raises(B.BiError) as e:
        B.plan_query(B.BI_OP_RMSNORM, 4100, 0)
    assert e.value.status == B.BI_ERR_SHAPE
    with pytest.raises(B.BiError) as e:
        B.plan_query(B.BI_OP_RMSNORM, 65536, 0)
    assert e.value.status == B.BI_ERR_UNSUPPORTED
    with pytest.raises(B.BiError):
        B.plan_query(99, 256, 512)


def test_rmsnorm_plan():
    p = B.plan_query(B.BI_OP_RMSNORM, 512, 0)
    assert p["threads"] == 64 and p["chunks_per_thread"] == 1
    p = B.plan_query(B.BI_OP_RMSNORM, 4096, 0)
    assert p["threads"] == 256 and p["chunks_per_thread"] == 2


A0, B0, Y0 = 0x10000, 0x200000, 0x4000000   # fake, 16-byte aligned, disjoint


def gemm(A=A0, lda=512, Bp=B0, ldb=512, Y=Y0, ldy=256, M=4, N=256, K=512):
    return B.lib().bi_gemm(A, lda, Bp, ldb, Y, ldy, M, N, K, None)


def test_gemm_validation():
    assert gemm(M=-1) == B.BI_ERR_SHAPE
    assert gemm(K=12, lda=16, ldb=16) == B.BI_ERR_SHAPE
    assert gemm(lda=256) == B.BI_ERR_SHAPE
    assert gemm(ldy=100) == B.BI_ERR_SHAPE
    assert gemm(N=0) == B.BI_ERR_SHAPE
    assert gemm(A=0) == B.BI_ERR_NULL
    assert gemm(Y=0) == B.BI_ERR_NULL
    assert gemm(A=A0 + 2) == B.BI_ERR_ALIGN
    assert gemm(lda=516) == B.BI_ERR_ALIGN
    assert gemm(Y=A0 + 16) == B.BI_ERR_ALIAS
    assert gemm(Y=B0 + 4096) == B.BI_ERR_ALIAS
    # M == 0 is a no-op, even with NULL pointers
    assert gemm(M=0, A=0, Bp=0, Y=0) == B.BI_OK


def test_bmm_validation():
    f = B.lib().bi_bmm
    # A [2,4,128], B [2,128,512], Y [2,4,512]
    ok = dict(A=A0, sA=512, lda=128, B=B0, sB=65536, ldb=512, Y=Y0, sY=2048, ldy=512,
              batch=2, M=4, N=512, K=128)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["A"], a["sA"], a["lda"], a["B"], a["sB"], a["ldb"], a["Y"], a["sY"], a["ldy"],
                 a["batch"], a["M"], a["N"], a["K"], None)
    assert call(N=500, ldb=500, ldy=500) == B.BI_ERR_SHAPE
    assert call(batch=0) == B.BI_ERR_SHAPE
    assert call(sA=100) == B.BI_ERR_SHAPE
    assert call(Y=0) == B.BI_ERR_NULL
    assert call(Y=B0 + 16) == B.BI_ERR_ALIAS
    assert call(M=0, A=0, B=0, Y=0) == B.BI_OK


def test_nvfp4_validation():
    f = B.lib().bi_nvfp4_gemm

    def call(A=A0, As=0, fmt=0, lda=4096, W=B0, Ws=B0 + 0x1000000, alpha=1.0, Y=Y0, ldy=256,
             M=4, N=256, K=4096):
        return f(A, As, fmt, lda, W, Ws, alpha, Y, ldy, M, N, K, None)
    assert call(K=4080, lda=4080) == B.BI_ERR_SHAPE
    assert call(fmt=7) == B.BI_ERR_SHAPE
    assert call(fmt=1) == B.BI_ERR_NULL           # NVFP4 A needs scales
    assert call(Ws=0) == B.BI_ERR_NULL
    assert call(fmt=1, As=0x3000000, lda=4104) == B.BI_ERR_ALIGN
    assert call(Y=B0 + 64) == B.BI_ERR_ALIAS
    assert call(M=0, A=0, W=0, Ws=0, Y=0) == B.BI_OK


def test_rmsnorm_validation():
    f = B.lib().bi_rmsnorm

    def call(X=A0, ldx=4096, g=B0, eps=1e-6, Y=Y0, ldy=4096, M=4, H=4096):
        return f(X, ldx, g, eps, Y, ldy, M, H, None)
    assert call(H=4100, ldx=4104, ldy=4104) == B.BI_ERR_SHAPE
    assert call(H=65536, ldx=65536, ldy=65536) == B.BI_ERR_UNSUPPORTED
    assert call(g=0) == B.BI_ERR_NULL
    assert call(Y=A0 + 32) == B.BI_ERR_ALIAS      # partial overlap with X
    assert call(Y=B0) == B.BI_ERR_ALIAS           # overlaps gamma
    assert call(M=0, X=0, g=0, Y=0) == B.BI_OK


def test_nvfp4_quant_plan():
    p = B.plan_query(B.BI_OP_NVFP4_QUANT, 4096, 0)
    assert p["threads"] == 256 and p["chunks_per_thread"] == 1
    with pytest.raises(B.BiError) as e:
        B.plan_query(B.BI_OP_NVFP4_QUANT, 4104, 0)
    assert e.value.status == B.BI_ERR_SHAPE


def test_nvfp4_quant_validation():
    f = B.lib().bi_nvfp4_quant

    def call(X=A0, ldx=4096, g=2.5, Q=B0, S=B0 + 0x100000, ldq=4096, M=4, K=4096):
        return f(X, ldx, g, Q, S, ldq, M, K, None)
    assert call(K=4088, ldx=4088, ldq=4096) == B.BI_ERR_SHAPE      # K % 16
    assert call(ldx=4080) == B.BI_ERR_SHAPE                        # ldx < K
    assert call(ldq=4080) == B.BI_ERR_SHAPE                        # ldq < K
    assert call(M=-1) == B.BI_ERR_SHAPE
    for bad_g in (0.0, -1.0, float("nan"), float("inf")):
        assert call(g=bad_g) == B.BI_ERR_VALUE, bad_g
    assert call(X=0) == B.BI_ERR_NULL
    assert call(S=0) == B.BI_ERR_NULL
    assert call(ldq=4104) == B.BI_ERR_ALIGN                        # ldq % 16
    assert call(ldx=4100) == B.BI_ERR_ALIGN                        # ldx % 8
    assert call(X=A0 + 8) == B.BI_ERR_ALIGN
    assert call(Q=B0 + 2) == B.BI_ERR_ALIGN
    assert call(Q=A0 + 64) == B.BI_ERR_ALIAS                       # codes over X
    assert call(S=B0 + 64) == B.BI_ERR_ALIAS                       # scales over codes
    assert call(M=1 << 20, K=8192, ldx=8192, ldq=8192) == B.BI_ERR_UNSUPPORTED
    assert call(M=0, X=0, Q=0, S=0) == B.BI_OK


def test_reduce_rmsnorm_plan_matches_rmsnorm():
    for H in (512, 4096, 1000):
        assert B.plan_query(B.BI_OP_REDUCE_RMSNORM, H, 0)["threads"] == B.plan_query(B.BI_OP_RMSNORM, H, 0)["threads"]


def test_reduce_rmsnorm_validation():
    f = B.lib().bi_reduce_rmsnorm
    P0, P1, RES, G, R, Y = 0x10000000, 0x11000000, 0x12000000, 0x13000000, 0x14000000, 0x15000000

    def call(parts=(P0, P1), n=None, ldp=4096, res=RES, ldres=4096, g=G, R=R, ldr=4096, Y=Y,
             ldy=4096, M=4, H=4096):
        arr = (ctypes.c_void_p * max(1, len(parts)))(*parts) if parts is not None else None
        return f(arr, len(parts) if n is None else n, ldp, res, ldres, g, 1e-6, R, ldr, Y, ldy, M, H, None)
    assert call(n=0) == B.BI_ERR_SHAPE
    assert call(parts=(P0,) * 9) == B.BI_ERR_SHAPE              # more than 8 partials
    assert call(H=4100, ldp=4104, ldres=4104, ldr=4104, ldy=4104) == B.BI_ERR_SHAPE
    assert call(ldp=2048) == B.BI_ERR_SHAPE
    assert call(H=65536, ldp=65536, ldres=65536, ldr=65536, ldy=65536) == B.BI_ERR_UNSUPPORTED
    assert call(parts=(P0, 0)) == B.BI_ERR_NULL
    assert call(Y=0) == B.BI_ERR_NULL
    assert call(parts=(P0, P1 + 8)) == B.BI_ERR_ALIGN
    assert call(res=RES + 8) == B.BI_ERR_ALIGN
    assert call(R=P1 + 64) == B.BI_ERR_ALIAS                     # R over a partial
    assert call(Y=R + 1024) == B.BI_ERR_ALIAS                    # Y over R
    assert call(Y=RES) == B.BI_ERR_ALIAS                         # Y over the residual
    assert call(R=RES + 64) == B.BI_ERR_ALIAS                    # partial overlap with the residual
    assert call(res=0, ldres=0, M=0) == B.BI_OK
    assert call(parts=(0, 0), M=0, g=0, R=0, Y=0) == B.BI_OK


def test_grouped_gemm_plan_shares_the_gemm_chain():
    """The grouped GEMM's tile may differ from the dense one (every tile shape
    gives the same bits), but the MFMA block and K step are the same.  The
    tile follows N and the average rows per expert: 128 x 128 up to 96 rows,
    256 x 128 to 192, 256 x 192 to 768, then 256 x 256 (N >= 2048); 128 x 128
    for 512 <= N < 2048 and 64 x 64 below."""
    for N, K in ((6144, 4096), (4096, 4096), (1536, 4096), (256, 1024)):
        g, q = B.plan_query(B.BI_OP_GEMM, N, K), B.plan_query(B.BI_OP_GROUPED_GEMM, N, K)
        for key in ("mfma_m", "mfma_n", "mfma_k", "bk"):
            assert g[key] == q[key]
        assert q == B.plan_query(B.BI_OP_GROUPED_GEMM, N, K)
    assert B.plan_query(B.BI_OP_GROUPED_GEMM, 4096, 4096)["bn"] == 256
    shapes = B.tile_shapes()

    def bands(N):
        return [(r["m_min"], r["m_max"], shapes[r["tile_variant"] - 1]["bm"], shapes[r["tile_variant"] - 1]["bn"])
                for r in B.plan_regimes(B.BI_OP_GROUPED_GEMM, N, 4096, cus=256)]
    big = 2 ** 31 - 1
    assert bands(4096) == [(1, 96, 128, 128), (97, 192, 256, 128), (193, 768, 256, 192), (769, big, 256, 256)]
    assert bands(1536) == [(1, big, 128, 128)]
    assert bands(256) == [(1, big, 64, 64)]


def test_grouped_gemm_validation():
    f = B.lib().bi_grouped_gemm
    OFF = 0x7000000

    def call(A=A0, lda=512, W=B0, ldw=512, sW=256 * 512, Y=Y0, ldy=256, off=OFF, E=4, T=40, N=256, K=512):
        return f(A, lda, W, ldw, sW, Y, ldy, off, E, T, N, K, None)
    assert call(E=0) == B.BI_ERR_SHAPE
    assert call(K=12, lda=16, ldw=16) == B.BI_ERR_SHAPE
    assert call(sW=1000) == B.BI_ERR_SHAPE                       # experts overlap
    assert call(T=-1) == B.BI_ERR_SHAPE
    assert call(off=0) == B.BI_ERR_NULL
    assert call(off=OFF + 4) == B.BI_ERR_ALIGN
    assert call(A=A0 + 8) == B.BI_ERR_ALIGN
    assert call(Y=B0 + 64) == B.BI_ERR_ALIAS                     # Y over an expert weight
    assert call(Y=A0 + 1024) == B.BI_ERR_ALIAS
    assert call(T=0, A=0, W=0, Y=0, off=0) == B.BI_OK


def test_mla_decode_validation():
    f = B.lib().bi_mla_decode
    Q0, KV0, LN0, O0 = 0x1000000, 0x2000000, 0x6000000, 0x7000000

    def call(q=Q0, kv=KV0, lens=LN0, scale=0.04, out=O0, Bn=4, H=16, Lmax=1024, Dqk=576, Dv=512, ws=None,
             wsb=0):
        return f(q, kv, lens, scale, out, Bn, H, Lmax, Dqk, Dv, ws, wsb, None)
    assert call(Dqk=572) == B.BI_ERR_SHAPE                      # Dqk % 8
    assert call(Dv=500) == B.BI_ERR_SHAPE                       # Dv % 8
    assert call(Dv=584) == B.BI_ERR_SHAPE                       # Dv > Dqk
    assert call(Bn=-1) == B.BI_ERR_SHAPE
    assert call(Lmax=-1) == B.BI_ERR_SHAPE
    assert call(Dqk=1032, Dv=512) == B.BI_ERR_UNSUPPORTED
    assert call(Lmax=16385) == B.BI_ERR_UNSUPPORTED
    assert call(scale=float("nan")) == B.BI_ERR_VALUE
    assert call(scale=float("inf")) == B.BI_ERR_VALUE
    assert call(lens=0) == B.BI_ERR_NULL
    assert call(q=Q0 + 8) == B.BI_ERR_ALIGN
    assert call(lens=LN0 + 2) == B.BI_ERR_ALIGN
    assert call(out=Q0 + 1024) == B.BI_ERR_ALIAS                 # out over q
    assert call(out=KV0 + 4096) == B.BI_ERR_ALIAS                # out over the cache
    assert call(Bn=0, q=0, kv=0, lens=0, out=0) == B.BI_OK
    assert call(H=0, q=0, kv=0, lens=0, out=0) == B.BI_OK
    need = B.mla_decode_workspace_size(4, 16, 1024, 576, 512)
    assert need == 4 * 1 * 1 * (32 + 16 * 512) * 4                 # 1 chunk of 1024 tokens
    WS0 = 0x8000000
    assert call(ws=WS0, wsb=need - 4) == B.BI_ERR_SHAPE            # too small
    assert call(ws=WS0 + 8, wsb=need) == B.BI_ERR_ALIGN
    assert call(ws=KV0 + 4096, wsb=need) == B.BI_ERR_ALIAS          # over the cache
    assert call(ws=O0 - 64, wsb=need) == B.BI_ERR_ALIAS             # runs into out
    assert call(Bn=0, q=0, kv=0, lens=0, out=0, ws=WS0, wsb=need) == B.BI_OK
    # shapes served by the VALU kernel use no workspace
    assert B.mla_decode_workspace_size(4, 16, 1024, 1024, 1024) == 0
    assert B.mla_decode_workspace_size(4, 20, 5000, 576, 512) == 4 * 2 * 5 * (32 + 16 * 512) * 4
    with pytest.raises(B.BiError):
        B.mla_decode_workspace_size(4, 16, 1024, 572, 512)


def test_mla_decode_noalloc_validation():
    """The no-allocation decode entry point validates like bi_mla_decode
    before it touches the device or its scratch array."""
    f = B.lib().bi_mla_decode_noalloc
    Q0, KV0, LN0, O0 = 0x1000000, 0x2000000, 0x6000000, 0x7000000

    def call(q=Q0, kv=KV0, lens=LN0, scale=0.04, out=O0, Bn=4, H=16, Lmax=1024, Dqk=576, Dv=512):
        return f(q, kv, lens, scale, out, Bn, H, Lmax, Dqk, Dv, None)
    assert call(Dqk=572) == B.BI_ERR_SHAPE
    assert call(Dv=584) == B.BI_ERR_SHAPE
    assert call(Lmax=16385) == B.BI_ERR_UNSUPPORTED
    assert call(scale=float("nan")) == B.BI_ERR_VALUE
    assert call(lens=0) == B.BI_ERR_NULL
    assert call(q=Q0 + 8) == B.BI_ERR_ALIGN
    assert call(out=KV0 + 4096) == B.BI_ERR_ALIAS
    assert call(Bn=0, q=0, kv=0, lens=0, out=0) == B.BI_OK
    assert call(H=0, q=0, kv=0, lens=0, out=0) == B.BI_OK
    assert B.MLA_SCRATCH_BYTES == 32 << 20


@pytest.mark.parametrize("op,N,K,a_fmt", [(B.BI_OP_GEMM, 256, 512, 0), (B.BI_OP_GEMM, 6144, 4096, 0),
                                          (B.BI_OP_GEMM, 4096, 4096, 0), (B.BI_OP_GEMM, 24576, 4096, 0),
                                          (B.BI_OP_GEMM, 4096, 12288, 0), (B.BI_OP_NVFP4_GEMM, 24576, 4096, 0),
                                          (B.BI_OP_NVFP4_GEMM, 24576, 4096, 1), (B.BI_OP_NVFP4_GEMM, 1000, 4160, 0),
                                          (B.BI_OP_BMM, 512, 128, 0), (B.BI_OP_GROUPED_GEMM, 4096, 4096, 0)])
def test_plan_regimes_cover_every_m(op, N, K, a_fmt):
    """The kernel-choice table covers M >= 1 without gaps or overlaps; its
    last range starts by 4097 rows and is the tiled kernel of bi_plan_query's
    shape (or the streaming BMM kernel), unbounded above; streaming ranges
    end by 128 rows; every tiled range names a compiled shape that matches
    its row blocks and columns."""
    shapes = B.tile_shapes()
    for cus in (80, 256, 304):
        regs = B.plan_regimes(op, N, K, a_fmt, cus=cus)
        assert regs[0]["m_min"] == 1 and regs[-1]["m_max"] == 2 ** 31 - 1
        for a, b in zip(regs, regs[1:]):
            assert b["m_min"] == a["m_max"] + 1
            assert a != b
        last = regs[-1]
        plan = B.plan_query(op, N, K)
        if last["kind"] != "bmm_stream":
            assert last["kind"] in ("tiled", "tiled_pingpong")
            assert (last["row_blocks"] * 16, last["cols"]) == (plan["bm"], plan["bn"])
            assert last["m_min"] <= 4097
        for r in regs:
            if r["kind"].startswith("tiled"):
                t = shapes[r["tile_variant"] - 1]
                assert (t["bm"], t["bn"]) == (r["row_blocks"] * 16, r["cols"])
            else:
                assert r["tile_variant"] == 0
                assert r["kind"] == "bmm_stream" or r["m_max"] <= 128
        if op == B.BI_OP_GROUPED_GEMM:
            assert all(r["kind"] == "tiled" for r in regs)   # shapes by rows per expert
        if a_fmt == 1:
            # an NVFP4 A streams only through the A-in-LDS kernel (M <= 16)
            # and the chunked-A kernel (16 < M <= 128)
            assert all(r["kind"] == "tiled" or (r["kind"] == "stream_a_lds" and r["m_max"] <= 16) or
                       (r["kind"] == "stream_a_chunks" and 17 <= r["m_min"] and r["m_max"] <= 128) for r in regs)


def _shape_at(op, N, K, M, a_fmt=0, cus=256):
    for r in B.plan_regimes(op, N, K, a_fmt, cus=cus):
        if r["m_min"] <= M <= r["m_max"]:
            if r["kind"].startswith("tiled"):
                return (r["row_blocks"] * 16, r["cols"])
            return r["kind"]
    raise AssertionError(M)


def test_plan_regimes_cost_model_choices():
    """The kernel at each M of the Qwen3-8B-shaped linears on a 256-CU
    device (the tiled kernel's shape, or a streaming kernel) is the one the
    MI355X sweeps of every compiled shape and of the streaming kernels found
    fastest (or within a few percent of it)."""
    G, F = B.BI_OP_GEMM, B.BI_OP_NVFP4_GEMM
    want = {
        (G, 6144, 4096): {32: "stream_a_chunks", 64: "stream_a_chunks", 128: (64, 64), 256: (128, 64), 512: (128, 128), 1024: (256, 128),
                          2048: (256, 192), 4096: (256, 192), 8192: (256, 256)},
        (G, 4096, 4096): {32: "stream_reg", 64: "stream_reg", 128: (64, 64), 256: (64, 64), 512: (128, 64),
                          1024: (128, 128), 2048: (256, 128), 4096: (256, 256), 8192: (256, 256)},
        (G, 24576, 4096): {32: "stream_a_chunks", 64: "stream_a_chunks", 128: (128, 128), 256: (256, 128), 512: (256, 192),
                           1024: (256, 192), 2048: (256, 256), 4096: (256, 256)},
        (G, 4096, 12288): {32: "stream_reg", 64: "stream_reg", 128: (64, 64), 256: (64, 64), 512: (128, 64),
                           1024: (128, 128), 2048: (256, 128), 4096: (256, 256), 8192: (256, 256)},
        (F, 24576, 4096): {32: "stream_a_chunks", 64: "stream_a_chunks", 128: "stream_a_chunks", 256: (256, 128),
                           1024: (256, 192), 2048: (256, 256), 4096: (256, 256)},
    }
    for (op, N, K), ms in want.items():
        for M, shape in ms.items():
            assert _shape_at(op, N, K, M) == shape, (op, N, K, M)
    w4a4 = {32: "stream_a_chunks", 64: "stream_a_chunks", 128: "stream_a_chunks", 256: (256, 128), 512: (256, 192), 1024: (256, 192),
            2048: (256, 256), 4096: (256, 256)}
    for M, shape in w4a4.items():
        assert _shape_at(F, 24576, 4096, M, a_fmt=1) == shape, M
    for M in (1, 16):
        assert _shape_at(F, 24576, 4096, M, a_fmt=1) == "stream_a_lds", M


def test_plan_regimes_edges_and_errors():
    # the A-in-LDS limit 10 * M * cus <= 7 * N moves with the compute-unit count
    r = B.plan_regimes(B.BI_OP_GEMM, 4096, 4096, cus=256)
    assert (r[0]["kind"], r[0]["m_max"], r[1]["kind"]) == ("stream_a_lds", 11, "stream_reg")
    r = B.plan_regimes(B.BI_OP_GEMM, 4096, 4096, cus=128)
    assert (r[0]["kind"], r[0]["m_max"]) == ("stream_a_lds", 16)
    arr = (B.BiRegime * 1)()
    n = B.ctypes.c_int(0)
    st = B.lib().bi_plan_regimes(B.BI_OP_GEMM, 4096, 4096, 0, 256, arr, 1, B.ctypes.byref(n))
    assert st == B.BI_ERR_SHAPE and n.value == len(B.plan_regimes(B.BI_OP_GEMM, 4096, 4096, cus=256)) > 1
    assert B.lib().bi_plan_regimes(B.BI_OP_RMSNORM, 4096, 0, 0, 256, arr, 1, B.ctypes.byref(n)) == B.BI_ERR_UNSUPPORTED
    assert B.lib().bi_plan_regimes(B.BI_OP_GEMM, 4096, 4096, 1, 256, arr, 1, B.ctypes.byref(n)) == B.BI_ERR_SHAPE
    assert B.lib().bi_plan_regimes(B.BI_OP_GEMM, 4096, 4100, 0, 256, arr, 1, B.ctypes.byref(n)) == B.BI_ERR_SHAPE


def test_launch_opts_layout():
    """bi_launch_opts keeps its 32-byte layout (fixed_plan took a reserved
    slot), with the fields at the offsets bi.h gives them."""
    O = B.BiLaunchOpts
    assert B.ctypes.sizeof(O) == 32
    assert [O.max_workgroups.offset, O.tile_variant.offset, O.pipeline_depth.offset, O.fixed_plan.offset] == [0, 4, 8, 12]


def test_probe_validation():
    """The measurement probes validate their arguments before any launch."""
    L = B.lib()
    assert L.bi_probe_mfma(None, 10, 4, None) == B.BI_ERR_NULL
    assert L.bi_probe_mfma(0x1000, 0, 4, None) == B.BI_ERR_SHAPE
    assert L.bi_probe_mfma(0x1000, 10, 0, None) == B.BI_ERR_SHAPE
    assert L.bi_probe_mfma(0x1004, 10, 4, None) == B.BI_ERR_ALIGN
    assert L.bi_probe_read(0x1000, 0, 0x9000, 4, None) == B.BI_ERR_SHAPE
    assert L.bi_probe_read(0x1000, 24, 0x9000, 4, None) == B.BI_ERR_SHAPE
    assert L.bi_probe_read(0x1008, 1024, 0x9000, 4, None) == B.BI_ERR_ALIGN
    assert L.bi_probe_read(0x1000, 1 << 20, 0x2000, 4, None) == B.BI_ERR_ALIAS
    assert L.bi_probe_read(None, 1024, 0x9000, 4, None) == B.BI_ERR_NULL
    assert L.bi_probe_lds(None, 10, 4, None) == B.BI_ERR_NULL
    assert L.bi_probe_lds(0x1000, 0, 4, None) == B.BI_ERR_SHAPE
    assert L.bi_probe_lds(0x1000, 10, 0, None) == B.BI_ERR_SHAPE
    assert L.bi_probe_lds(0x1004, 10, 4, None) == B.BI_ERR_ALIGN
