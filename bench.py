"""Benchmark of the batch-invariant hot path on one MI355X.

One step = one pass of every operation of the path over one batch of
synthetic, seeded inputs already resident in HBM, shaped like a Qwen3-8B
decoder layer at M tokens (default M = 2048):
    RMSNorm(H=4096) -> qkv GEMM (N=6144, K=4096) -> MLA-absorbed BMM
    (128 heads, [M_b,128] . [128,512], M_b = min(M, 1024)) -> o_proj GEMM
    (4096, 4096) -> RMSNorm -> gate_up GEMM (24576, 4096) -> down GEMM
    (4096, 12288) -> NVFP4 gate_up GEMM (W[24576,4096] e2m1 + e4m3/16).
Activations ~ N(0,1), weights ~ N(0,0.02), rounded to bf16; the NVFP4
weight is the host quantisation of N(0,0.02) values; gamma ~ U(0.5,1.5).

Prints one JSON line:
  * `value`: the step's GEMM-family TFLOP/s (all flops of the step over the
    wall time of the timed steps, synchronised on both sides); each step is
    one replay of a HIP graph of the step's library calls, so no host
    launch cost sits between its kernels (the replayed outputs are checked
    bitwise against the eager step's);
  * `per_op`: every op of the step, its mean launch time from HIP events
    around replays of a graph of 20 launches of that op (on the stream the
    library launches on), and its fraction of the roofline max(bytes /
    8 TB/s, flops / 2.5 PFLOP/s) of its algorithmic work;
  * `roofline`: the longest op of the step; `traffic` is its HBM bytes per
    launch from the committed counter summary in profiles/ when that was
    taken with the current kernel sources, else null;
  * `ceilings`: what the machine measures under this benchmark -- an
    MFMA-only loop of the hot path's instruction (with the clock it ran
    at) and a 2 GiB read stream -- and each op's fraction of those;
  * `sweep`: every configuration of the metric over its M sweep (tiny GEMM,
    the Qwen3-8B linears 1..2048, long-K down_proj 1..8192 with 7/129/1000,
    the MLA-absorbed BMM, the NVFP4 weight with bf16 and with NVFP4
    activations 1..4096, RMSNorm), each point with its roofline fraction and
    a bitwise check of its rows against the largest M's; at M <= 256 the
    weights rotate over >= 1 GiB of copies so that the last-level cache
    cannot serve them; plus the next-row operations (quantiser, reduction +
    RMSNorm, grouped GEMM, MLA decode);
  * `invariance`: bitwise checks passed / made;
  * `cpu_baseline`: the fp64 oracle timed on a bounded sample of the step.

Profiler passes (run under rocprofv3; see profiles/):
    python bench.py --only-step --calib --steps 5 --warmup 2
and their summary:
    python bench.py --summarize <rocprofv3 output dir(s)> --kernel <name> --out <file>
"""
import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CALIB_BYTES = 512 << 20     # bytes read by the calibration read stream (and copied once)
# counter summaries, keyed by the step op they cover
COUNTER_FILES = {
    "nvfp4_gate_up": os.path.join(ROOT, "profiles", "gemm_nvfp4_gate_up_M2048_counters.txt"),
    "gate_up": os.path.join(ROOT, "profiles", "gemm_gate_up_M2048_counters.txt"),
}
TRACE_FILE = os.path.join(ROOT, "profiles", "bench_step_M2048_kernel_trace.txt")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--m", type=int, default=2048, help="tokens per step")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    p.add_argument("--only-step", action="store_true", help="run the timed steps only (for profiler passes)")
    p.add_argument("--only-mla", action="store_true",
                   help="run the MLA decode next-row workload only (workspace schedule; for profiler passes)")
    p.add_argument("--calib", action="store_true",
                   help="after the steps, read 512 MiB three times and copy 512 MiB three times "
                        "(counter calibration)")
    p.add_argument("--w4a4", action="store_true",
                   help="after the steps, quantise the gate_up input and run the W4A4 GEMM three times "
                        "(untimed; for profiler passes)")
    p.add_argument("--summarize", metavar="DIR", nargs="+", help="summarise rocprofv3 CSV output in DIR(s)")
    p.add_argument("--kernel", default="", help="kernel-name substring whose traffic --summarize reports")
    p.add_argument("--out", metavar="FILE", help="where --summarize writes its summary")
    p.add_argument("--command", default="", help="command line recorded by --summarize")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of the HIP/C++ sources: a profile summary is valid only for them."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "invariant_deterministic_bi_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".h", ".hip", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def read_summary(path):
    """key: value lines of a summary written by --summarize, or None when it
    is missing or was taken with other kernel sources."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    return kv


def roof(nbytes, flops):
    """(roofline time in us, bound) of one call's algorithmic work."""
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9) * 1e6
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12) * 1e6
    return (t_mfma, "mfma") if t_mfma >= t_hbm else (t_hbm, "hbm")


# ------------------------------------------------------------------ summaries

def summarize(dirs, out, command, kernel):
    """Condense rocprofv3 CSV output (kernel trace, counters) into text.

    Kernel trace: per (kernel, grid size) the calls, median, mean and min
    duration.  Counters: per (kernel, grid size) the mean per dispatch.
    HBM bytes come from the TCC read requests split by size (32, 64 and 128
    bytes) and the write requests (64 bytes, the rest 32): bytes = sum of
    size x count.  They are checked against kernels of known traffic -- the
    read probe (it reads CALIB_BYTES once) and a copy (it writes CALIB_BYTES)
    -- and the ratio is reported.  traffic_bytes_per_launch is the read +
    write bytes of the dispatches of `kernel` with the largest grid.
    """
    # the profiler's output folders, named by their last component
    lines = [f"# rocprofv3 summary written by: python bench.py --summarize "
             f"{' '.join('<out>/' + os.path.basename(os.path.normpath(d)) for d in dirs)}"
             + (f" --kernel {kernel}" if kernel else ""),
             f"# profiled command(s): {command}" if command else "#",
             f"kernel_source_sha: {kernel_source_sha()}"]
    acc = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            every = {}
            for r in csv.DictReader(open(path)):
                g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                every.setdefault((r["Kernel_Name"][:110], g), []).append(dur)
            if every:
                lines.append("# kernel trace, per kernel and grid size (threads), largest total first: "
                             "name | grid | calls | median ns | mean ns | min ns")
                for (n, g), v in sorted(every.items(), key=lambda kv: -sum(kv[1])):
                    if "bi::" not in n:
                        continue
                    lines.append(f"{n} | {g} | {len(v)} | {statistics.median(v):.0f} | {sum(v) / len(v):.0f} | "
                                 f"{min(v)}")
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                key = (r["Kernel_Name"][:110], int(r["Grid_Size"]), r["Counter_Name"])
                acc.setdefault(key, []).append(float(r["Counter_Value"]))
    if acc:
        mean = {k: sum(v) / len(v) for k, v in acc.items()}
        lines.append("# counters, mean per dispatch, for this library's kernels and the two calibration kernels: "
                     "name | grid | counter | value | dispatches")
        for (n, g, c), m in sorted(mean.items()):
            if "bi::" in n or "direct_copy" in n:
                lines.append(f"{n} | {g} | {c} | {m:.1f} | {len(acc[(n, g, c)])}")

        def bytes_of(n, g):
            r32, r64, r128 = (mean.get((n, g, f"TCC_EA0_RDREQ_{s}B")) for s in (32, 64, 128))
            rd = None if None in (r32, r64, r128) else 32.0 * r32 + 64.0 * r64 + 128.0 * r128
            w, w64 = mean.get((n, g, "TCC_EA0_WRREQ")), mean.get((n, g, "TCC_EA0_WRREQ_64B"))
            wr = None if None in (w, w64) else 64.0 * w64 + 32.0 * (w - w64)
            return rd, wr

        names = sorted({(n, g) for (n, g, _) in mean})
        for n, g in names:
            rd, wr = bytes_of(n, g)
            if "read_probe_kernel" in n and rd is not None:
                lines.append(f"read_probe_bytes_measured_over_true: {rd / CALIB_BYTES:.4f}")
            if "direct_copy" in n and wr is not None:
                lines.append(f"copy_write_bytes_measured_over_true: {wr / CALIB_BYTES:.4f}")
        if kernel:
            cand = [(g, n) for (n, g) in names if kernel in n]
            if cand:
                g, n = max(cand)
                rd, wr = bytes_of(n, g)
                lines.append(f"traffic_kernel: {n}")
                lines.append(f"traffic_grid_threads: {g}")
                if rd is not None:
                    lines.append(f"traffic_read_bytes_per_launch: {rd:.0f}")
                if wr is not None:
                    lines.append(f"traffic_write_bytes_per_launch: {wr:.0f}")
                if rd is not None and wr is not None:
                    lines.append(f"traffic_bytes_per_launch: {rd + wr:.0f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------------ main

def mla_only(args, B, inputs, np, torch, dev):
    """The MLA decode next row's workload (64 requests of 1024-4096 tokens,
    16 heads, 576/512, with the workspace), the same seeded inputs as the
    sweep, called `steps` times after `warmup` calls; one JSON line with the
    mean of HIP events around the timed calls."""
    gen = torch.Generator(device=dev)

    def randn(shape, std, seed):
        gen.manual_seed(seed)
        return torch.randn(shape, generator=gen, device=dev).mul_(std).to(torch.bfloat16)

    Bq, Hq, Dqk, Dv, Lmx = 64, 16, 576, 512, 4096
    lens_np = inputs.rng(12345, 21).integers(1024, Lmx + 1, Bq).astype(np.int32)
    qa = randn((Bq, Hq, Dqk), 1.0, 90)
    kva = randn((Bq, Lmx, Dqk), 1.0, 91)
    lens_d = torch.from_numpy(lens_np).to(dev)
    wsa = torch.empty(B.mla_decode_workspace_size(Bq, Hq, Lmx, Dqk, Dv), dtype=torch.uint8, device=dev)
    sc = 1.0 / 192 ** 0.5
    oa = B.bi_mla_decode(qa, kva, lens_d, sc, Dv, workspace=wsa)
    for _ in range(args.warmup):
        B.bi_mla_decode(qa, kva, lens_d, sc, Dv, oa, workspace=wsa)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        B.bi_mla_decode(qa, kva, lens_d, sc, Dv, oa, workspace=wsa)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    print(json.dumps({"metric": "mla_decode", "us_per_call": round(us, 2), "tokens": int(lens_np.sum()),
                      "GB/s": round((2.0 * int(lens_np.sum()) * Dqk) / (us * 1e-6) / 1e9, 1)}), flush=True)


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.out or os.path.join(args.summarize[0], "summary.txt"), args.command,
                  args.kernel)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the batch-invariant path here is single-GPU "
              "(no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from invariant_deterministic_bi_amd import binding as B
    from invariant_deterministic_bi_amd import inputs

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if args.only_mla:
        mla_only(args, B, inputs, np, torch, dev)
        return
    M = args.m
    Mb = min(M, 1024)
    H, Nqkv, No, Ngu, Kdn, heads, dk, dn = 4096, 6144, 4096, 24576, 12288, 128, 128, 512
    eps = 1e-6

    def d(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    t0 = time.time()
    log(f"generating inputs M={M}")
    host = {
        "X": inputs.randn_bf16((M, H), 1.0, tag=(1,)),
        "X2": inputs.randn_bf16((M, H), 1.0, tag=(2,)),
        "g1": inputs.uniform_bf16((H,), 0.5, 1.5, tag=(3,)),
        "g2": inputs.uniform_bf16((H,), 0.5, 1.5, tag=(4,)),
        "Wqkv": inputs.randn_bf16((Nqkv, H), 0.02, tag=(5,)),
        "Amla": inputs.randn_bf16((heads, Mb, dk), 1.0, tag=(6,)),
        "Bmla": inputs.randn_bf16((heads, dk, dn), 1.0, tag=(7,)),
        "Ao": inputs.randn_bf16((M, H), 1.0, tag=(8,)),
        "Wo": inputs.randn_bf16((No, H), 0.02, tag=(9,)),
        "Wgu": inputs.randn_bf16((Ngu, H), 0.02, tag=(10,)),
        "Adn": inputs.randn_bf16((M, Kdn), 1.0, tag=(11,)),
        "Wdn": inputs.randn_bf16((H, Kdn), 0.02, tag=(12,)),
    }
    w4_real = inputs.rng(12345, 13).standard_normal((Ngu, H)).astype(np.float32) * np.float32(0.02)
    g4 = inputs.nvfp4_global_scale(w4_real)
    host["W4"], host["W4s"] = inputs.nvfp4_quantize(w4_real, g4)
    del w4_real
    alpha4 = float(np.float32(1.0) / g4)
    t = {k: d(v) for k, v in host.items()}
    log(f"inputs ready in {time.time() - t0:.1f}s")

    out = {
        "Xn": torch.empty((M, H), dtype=torch.bfloat16, device=dev),
        "Xn2": torch.empty((M, H), dtype=torch.bfloat16, device=dev),
        "Yqkv": torch.empty((M, Nqkv), dtype=torch.bfloat16, device=dev),
        "Ymla": torch.empty((heads, Mb, dn), dtype=torch.bfloat16, device=dev),
        "Yo": torch.empty((M, No), dtype=torch.bfloat16, device=dev),
        "Ygu": torch.empty((M, Ngu), dtype=torch.bfloat16, device=dev),
        "Ydn": torch.empty((M, H), dtype=torch.bfloat16, device=dev),
        "Y4": torch.empty((M, Ngu), dtype=torch.bfloat16, device=dev),
    }

    def gemm_work(m, n, k):
        return 2.0 * (m * k + n * k + m * n), 2.0 * m * n * k

    def nvfp4_work(m, n, k, a_fp4=False):
        a_bytes = m * k / 2 + m * k / 16 if a_fp4 else 2.0 * m * k
        return a_bytes + n * k / 2 + n * k / 16 + 2.0 * m * n, 2.0 * m * n * k

    # the step: (name, launch, (algorithmic bytes, flops), kernel-name substring in rocprof output)
    ops = [
        ("rmsnorm_in", lambda: B.bi_rmsnorm(t["X"], t["g1"], eps, out["Xn"]), (4.0 * M * H + 2.0 * H, 4.0 * M * H),
         "rmsnorm_kernel"),
        ("qkv", lambda: B.bi_gemm(out["Xn"], t["Wqkv"], out["Yqkv"]), gemm_work(M, Nqkv, H), "pingpong_kernel<192>"),
        ("mla_bmm", lambda: B.bi_bmm(t["Amla"], t["Bmla"], out["Ymla"]),
         (2.0 * heads * (Mb * dk + dk * dn + Mb * dn), 2.0 * heads * Mb * dn * dk), "bmm"),
        ("o_proj", lambda: B.bi_gemm(t["Ao"], t["Wo"], out["Yo"]), gemm_work(M, No, H), "gemm_kernel<256, 128"),
        ("rmsnorm_post", lambda: B.bi_rmsnorm(t["X2"], t["g2"], eps, out["Xn2"]),
         (4.0 * M * H + 2.0 * H, 4.0 * M * H), "rmsnorm_kernel"),
        ("gate_up", lambda: B.bi_gemm(out["Xn2"], t["Wgu"], out["Ygu"]), gemm_work(M, Ngu, H), "pingpong_kernel<256>"),
        ("down", lambda: B.bi_gemm(t["Adn"], t["Wdn"], out["Ydn"]), gemm_work(M, H, Kdn), "gemm_kernel<256, 128"),
        ("nvfp4_gate_up", lambda: B.bi_nvfp4_gemm(out["Xn2"], t["W4"], t["W4s"], alpha4, out["Y4"]),
         nvfp4_work(M, Ngu, H), "pingpong_nvfp4_kernel"),
    ]
    step_flops = sum(w[1] for (n, _, w, _) in ops if not n.startswith("rmsnorm"))

    def step():
        for _, fn, _, _ in ops:
            fn()

    def capture(fn, reps):
        """A HIP graph of `reps` back-to-back calls of fn on a side stream (the
        library launches on torch's current stream, so its kernels are
        captured; it allocates nothing and never synchronises)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        return g

    def graph_us(fn, reps, replays=3, warm_ms=40.0):
        """Mean time of one call, from HIP events around `replays` replays of
        a graph of `reps` calls (no host launch cost between the kernels).
        The graph is first replayed, untimed, for at least `warm_ms`: the
        GPU's clock settles over the first tens of milliseconds of a new
        sustained load (a qkv call measured 106 us in the second replay and
        85-90 us from the fifth on)."""
        g = capture(fn, reps)
        t_w = time.perf_counter()
        n_w = 0
        while n_w < 2 or (time.perf_counter() - t_w) * 1e3 < warm_ms:
            g.replay()
            torch.cuda.synchronize()
            n_w += 1
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * replays)

    # eager step first: its outputs are the reference for the graph replays
    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    step_graph = capture(step, 1)
    for _ in range(args.warmup):
        step_graph.replay()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps (graph replays of one step)")
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step_graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t1
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    replay_equal = {k: bool(torch.equal(out[k], eager[k])) for k in out}
    op_us = {}
    for name, fn, _, _ in ops:
        op_us[name] = graph_us(fn, 20)
    log(f"step {ms_per_step:.3f} ms, {value:.1f} TFLOP/s; " +
        ", ".join(f"{n} {op_us[n]:.1f} us" for n, _, _, _ in ops))
    if args.calib:
        # counter calibration: a read stream of known bytes (16-byte loads) and
        # a plain copy (bf16 -> fp16 conversion, its own kernel name)
        src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        sink = torch.empty(cus * 16 * 256, dtype=torch.int32, device=dev)
        dst = torch.empty(CALIB_BYTES // 2, dtype=torch.float16, device=dev)
        for _ in range(3):
            B.bi_probe_read(src, cus * 16, sink)
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration reads and copies of {CALIB_BYTES} bytes done")
    if args.w4a4:
        ga_ = inputs.nvfp4_global_scale(inputs.bf16_bits_to_f32(host["X2"]))
        q_, qs_ = B.bi_nvfp4_quant(out["Xn2"], ga_)
        for _ in range(3):
            B.bi_nvfp4_gemm(q_, t["W4"], t["W4s"], float(np.float32(1.0) / (np.float32(ga_) * np.float32(g4))),
                            out["Y4"], A_scales=qs_)
        torch.cuda.synchronize()
        log("W4A4 launches done")
    if args.only_step:
        print(json.dumps({"metric": "step", "ms_per_step": ms_per_step, "value": value,
                          "per_op_us": {n: round(v, 2) for n, v in op_us.items()}}), flush=True)
        return

    # ---------------------------------------------------------------- ceilings
    log("ceilings: MFMA loop, read stream and LDS reads")
    mgrid, iters = 2 * cus, 20000
    pout = torch.empty((mgrid * B.PROBE_WAVES, 3), dtype=torch.int64, device=dev)
    runs = []
    for _ in range(3):
        us = graph_us(lambda: B.bi_probe_mfma(iters, mgrid, pout), 1, 1)
        o = pout.cpu().numpy()
        clk = float(np.median(o[:, 0].astype(np.float64) / (o[:, 1].astype(np.float64) / 1e8))) / 1e6
        runs.append((mgrid * B.PROBE_WAVES * iters * 8 * B.PROBE_MFMA_FLOPS / (us * 1e-6) / 1e12, clk))
    mfma_tf, mfma_clk = sorted(runs)[1]
    rbuf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(cus * 16 * 256, dtype=torch.int32, device=dev)
    read_gbs = rbuf.numel() / graph_us(lambda: B.bi_probe_read(rbuf, cus * 16, sink), 5) / 1e3
    del rbuf
    lds_iters = 2000
    lout = torch.empty((cus * B.PROBE_WAVES, 2), dtype=torch.int64, device=dev)
    for _ in range(2):
        B.bi_probe_lds(lds_iters, cus, lout)
    torch.cuda.synchronize()
    lcyc = lout.cpu().numpy()[:, 0].astype(np.float64).reshape(cus, B.PROBE_WAVES).max(axis=1)
    lds_bpc = float(np.median(B.PROBE_WAVES * lds_iters * B.PROBE_LDS_BYTES / lcyc))
    ceilings = {"mfma_loop_tflops": round(mfma_tf, 1), "mfma_loop_clock_mhz": round(mfma_clk),
                "mfma_loop_frac_of_spec": round(mfma_tf / PEAK_BF16_TFLOPS, 4),
                "read_stream_2GiB_gbs": round(read_gbs, 1),
                "read_stream_frac_of_spec": round(read_gbs / PEAK_HBM_GBS, 4),
                "lds_read_bytes_per_cycle_per_cu": round(lds_bpc, 1),
                "how": "bi_probe_mfma: grid 2x#CU x 8 waves x 20000 x 8 v_mfma_f32_16x16x32_bf16, median of 3, "
                       "clock = s_memtime cycles / s_memrealtime ticks; bi_probe_read: 2 GiB, 16-byte loads, mean of 5; "
                       "bi_probe_lds: #CU workgroups x 8 waves x 2000 x 16 conflict-free ds_read_b128, median over "
                       "workgroups of 8 x 2000 x 16 KB / the workgroup's largest cycle count"}
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True, text=True, timeout=30)
        if r.returncode == 0:
            ceilings["amd_smi_clock"] = json.loads(r.stdout)
    except Exception:  # amd-smi missing or slow: the probe's clock stands
        pass
    log(f"MFMA loop {mfma_tf:.0f} TFLOP/s at {mfma_clk:.0f} MHz; read stream {read_gbs:.0f} GB/s; "
        f"LDS reads {lds_bpc:.0f} B/cycle/CU")

    def frac_entry(name, us, work, launches):
        nbytes, flops = work
        t_roof, bound = roof(nbytes, flops)
        e = {"op": name, "us": round(us, 2), "bound": bound, "frac": round(t_roof / us, 4), "launches": launches}
        if bound == "mfma":
            e["TFLOP/s"] = round(flops / (us * 1e-6) / 1e12, 1)
            e["frac_of_measured_ceiling"] = round(flops / (us * 1e-6) / 1e12 / mfma_tf, 4)
        else:
            e["GB/s"] = round(nbytes / (us * 1e-6) / 1e9, 1)
            e["frac_of_measured_ceiling"] = round(nbytes / (us * 1e-6) / 1e9 / read_gbs, 4)
        return e

    per_op = [frac_entry(n, op_us[n], w, 60) for n, _, w, _ in ops]
    dom_i = max(range(len(ops)), key=lambda i: op_us[ops[i][0]])
    dname, _, dwork, dkernel = ops[dom_i]
    dus = op_us[dname]
    d_roof, d_bound = roof(*dwork)
    counters = read_summary(COUNTER_FILES.get(dname, ""))
    traffic = None
    if counters and dkernel in counters.get("traffic_kernel", ""):
        try:
            traffic = float(counters["traffic_bytes_per_launch"])
        except (KeyError, ValueError):
            traffic = None
    trace = read_summary(TRACE_FILE)
    trace_us = None
    if trace is not None:
        with open(TRACE_FILE) as f:
            for line in f:
                parts = [p.strip() for p in line.split("|")]
                if len(parts) == 6 and dkernel in parts[0] and int(parts[1]) > 0:
                    trace_us = round(float(parts[3]) / 1e3, 2)   # median ns
                    break
    achieved = dwork[1] / (dus * 1e-6) / 1e12 if d_bound == "mfma" else dwork[0] / (dus * 1e-6) / 1e9
    peak = PEAK_BF16_TFLOPS if d_bound == "mfma" else PEAK_HBM_GBS
    roofline = {"bound": d_bound, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s" if d_bound == "mfma" else "GB/s", "frac": round(achieved / peak, 4),
                "traffic": traffic, "op": dname, "kernel": dkernel,
                "per_launch_flops": dwork[1], "per_launch_algorithmic_bytes": dwork[0],
                "avg_launch_us": round(dus, 2), "launches_timed": 60,
                "timing": "HIP events around 3 replays of a graph of 20 launches, on the launch stream",
                "rocprof_median_us": trace_us,
                "frac_of_measured_ceiling": round(achieved / (mfma_tf if d_bound == "mfma" else read_gbs), 4)}

    result = {
        "metric": "batch-invariant GEMM TFLOP/s & GB/s vs M, % roofline; bitwise-invariance pass %",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, bf16; NVFP4 by host quantisation)",
        "config": {"workload": f"Qwen3-8B-shaped decoder-layer linears at M={M} tokens: rmsnorm(4096), "
                               f"qkv 6144x4096, MLA BMM 128x[{Mb},128]x[128,512], o_proj 4096x4096, "
                               f"rmsnorm, gate_up 24576x4096, down 4096x12288, NVFP4 gate_up 24576x4096",
                   "M": M, "global_batch": M, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "per_op": per_op,
        "ceilings": ceilings,
    }

    # ---------------------------------------------------------------- sweep
    inv = {"checked": 0, "passed": 0, "failed": []}

    def check(ok, what):
        inv["checked"] += 1
        inv["passed"] += int(bool(ok))
        if not ok:
            inv["failed"].append(what)

    for k, ok in replay_equal.items():
        check(ok, f"step graph replay == eager {k}")

    if not args.no_sweep:
        sweep = []
        fixed = []   # the fixed-plan option at a few M: context, not sweep points
        gen = torch.Generator(device=dev)

        def randn(shape, std, seed):
            gen.manual_seed(seed)
            return torch.randn(shape, generator=gen, device=dev).mul_(std).to(torch.bfloat16)

        def point(cfg, op, m, us, work, **extra):
            nbytes, flops = work
            t_roof, bound = roof(nbytes, flops)
            e = {"config": cfg, "op": op, "M": m, "us": round(us, 2), "bound": bound, "frac": float(f"{t_roof / us:.4g}"),
                 "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1), "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 2)}
            e.update(extra)
            sweep.append(e)
            return e

        def rotating(w_list, launch, m_small):
            """copies of the weight covering >= 1 GiB when m_small, else one"""
            return w_list if m_small else w_list[:1]

        def gemm_sweep(cfg, op, N, K, ms, wstd=0.02, seed=0, fixed_ms=()):
            W = randn((N, K), wstd, 1000 + seed)
            A = randn((max(ms), K), 1.0, 2000 + seed)
            Yfull = B.bi_gemm(A, W)
            ncopy = max(2, math.ceil((1 << 30) / (W.numel() * 2)))
            copies = [W] + [W.clone() for _ in range(ncopy - 1)]
            for m in ms:
                Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
                ws = rotating(copies, None, m <= 256)
                k = [0]

                def f():
                    B.bi_gemm(A[:m], ws[k[0] % len(ws)], Y)
                    k[0] += 1
                reps = max(50, 2 * len(ws)) if m <= 256 else 20
                us = graph_us(f, reps)
                B.bi_gemm(A[:m], W, Y)
                ok = torch.equal(Y, Yfull[:m])
                check(ok, f"{cfg} {op} M={m}")
                point(cfg, op, m, us, gemm_work(m, N, K), N=N, K=K, cold=m <= 256, bits_equal_full=ok)
                if m in fixed_ms:
                    # the same call with one tile shape per (N, K) at every M
                    def ff():
                        B.bi_gemm(A[:m], ws[k[0] % len(ws)], Y, fixed_plan=True)
                        k[0] += 1
                    fus = graph_us(ff, reps)
                    B.bi_gemm(A[:m], W, Y, fixed_plan=True)
                    okf = torch.equal(Y, Yfull[:m])
                    check(okf, f"{cfg} {op} M={m} fixed plan")
                    t_roof, _ = roof(*gemm_work(m, N, K))
                    fixed.append({"op": op, "M": m, "us": round(fus, 2), "default_us": round(us, 2),
                                  "frac": float(f"{t_roof / fus:.4g}"), "bits_equal_default": okf})
            del copies
            torch.cuda.empty_cache()

        log("sweep: tiny, Qwen3-8B linears, long-K down_proj")
        # tiny: A[M,512] . B[256,512]^T, every row alone as well
        W = randn((256, 512), 1.0, 11)
        A = randn((64, 512), 1.0, 12)
        Yfull = B.bi_gemm(A, W)
        for m in (1, 3, 7, 16, 64):
            Y = torch.empty((m, 256), dtype=torch.bfloat16, device=dev)
            us = graph_us(lambda: B.bi_gemm(A[:m], W, Y), 100)
            ok = torch.equal(Y, Yfull[:m])
            check(ok, f"tiny M={m}")
            point("C1 tiny", "gemm 256x512", m, us, gemm_work(m, 256, 512), bits_equal_full=ok,
                  note="launch-latency bound: time and invariance only")
        ys = torch.empty_like(Yfull)
        for i in range(64):
            B.bi_gemm(A[i:i + 1], W, ys[i:i + 1])
        check(torch.equal(ys, Yfull), "tiny every row alone")
        pow2 = [1 << i for i in range(12)]                      # 1 .. 2048
        for op, N in (("qkv", Nqkv), ("o_proj", No), ("gate_up", Ngu)):
            gemm_sweep("C2 Qwen3-8B linears", op, N, H, pow2, seed=N, fixed_ms=(1, 16, 128, 512))
        gemm_sweep("C3 down_proj long-K", "down", H, Kdn, sorted(set([1 << i for i in range(14)] + [7, 129, 1000])),
                   seed=7)

        log("sweep: BMM, NVFP4 (bf16 and NVFP4 activations), RMSNorm")
        Ab = randn((heads, 1024, dk), 1.0, 21)
        Bb = randn((heads, dk, dn), 1.0, 22)
        Yb = B.bi_bmm(Ab, Bb)
        for m in (1, 16, 128, 1024):
            Y = torch.empty((heads, m, dn), dtype=torch.bfloat16, device=dev)
            us = graph_us(lambda: B.bi_bmm(Ab[:, :m], Bb, Y), 50)
            ok = torch.equal(Y, Yb[:, :m])
            check(ok, f"bmm M={m}")
            point("C4 MLA-absorbed BMM", "bmm 128x[M,128]x[128,512]", m, us,
                  (2.0 * heads * (m * dk + dk * dn + m * dn), 2.0 * heads * m * dn * dk), bits_equal_full=ok)
        # NVFP4 weight: the step's W4 (host-quantised N(0,0.02)); A bf16 N(0,1) up to 4096 rows
        A4 = randn((4096, H), 1.0, 31)
        Y4full = B.bi_nvfp4_gemm(A4, t["W4"], t["W4s"], alpha4)
        ga = inputs.nvfp4_global_scale(A4.float().cpu().numpy())
        Aq, Aqs = B.bi_nvfp4_quant(A4, ga)
        alpha44 = float(np.float32(1.0) / (np.float32(ga) * np.float32(g4)))
        Y44full = B.bi_nvfp4_gemm(Aq, t["W4"], t["W4s"], alpha44, A_scales=Aqs)
        ncopy = 19
        w4c = [t["W4"]] + [t["W4"].clone() for _ in range(ncopy - 1)]
        s4c = [t["W4s"]] + [t["W4s"].clone() for _ in range(ncopy - 1)]
        for m in [1 << i for i in range(13)]:                   # 1 .. 4096
            n = ncopy if m <= 256 else 1
            Y = torch.empty((m, Ngu), dtype=torch.bfloat16, device=dev)
            for a_fp4 in (False, True):
                k = [0]

                def f():
                    j = k[0] % n
                    if a_fp4:
                        B.bi_nvfp4_gemm(Aq[:m], w4c[j], s4c[j], alpha44, Y, A_scales=Aqs[:m])
                    else:
                        B.bi_nvfp4_gemm(A4[:m], w4c[j], s4c[j], alpha4, Y)
                    k[0] += 1
                us = graph_us(f, max(50, 2 * n) if m <= 256 else 20)
                ref = Y44full if a_fp4 else Y4full
                if a_fp4:
                    B.bi_nvfp4_gemm(Aq[:m], t["W4"], t["W4s"], alpha44, Y, A_scales=Aqs[:m])
                else:
                    B.bi_nvfp4_gemm(A4[:m], t["W4"], t["W4s"], alpha4, Y)
                ok = torch.equal(Y, ref[:m])
                check(ok, f"nvfp4 {'w4a4' if a_fp4 else 'bf16 A'} M={m}")
                point("C5 NVFP4 weight", "nvfp4 w4a4" if a_fp4 else "nvfp4 bf16 A", m, us,
                      nvfp4_work(m, Ngu, H, a_fp4), cold=m <= 256, bits_equal_full=ok)
        del w4c, s4c
        for Hh, ms in ((4096, pow2), (512, (1, 3, 7, 16, 64))):
            X = randn((max(ms), Hh), 1.0, 40 + Hh)
            gam = (torch.rand((Hh,), generator=gen.manual_seed(50 + Hh), device=dev) + 0.5).to(torch.bfloat16)
            Yr = B.bi_rmsnorm(X, gam, eps)
            for m in ms:
                Y = torch.empty((m, Hh), dtype=torch.bfloat16, device=dev)
                us = graph_us(lambda: B.bi_rmsnorm(X[:m], gam, eps, Y), 50)
                ok = torch.equal(Y, Yr[:m])
                check(ok, f"rmsnorm H={Hh} M={m}")
                extra = {"note": "launch-latency bound: time and invariance only"} if (Hh == 512 or m <= 16) else {}
                point("RMSNorm", f"rmsnorm H={Hh}", m, us, (4.0 * m * Hh + 2.0 * Hh, 4.0 * m * Hh), bits_equal_full=ok,
                      **extra)

        log("sweep: next rows (quantiser, reduction + RMSNorm, grouped GEMM, MLA decode)")
        Aq2, Aqs2 = B.bi_nvfp4_quant(t["X2"], ga)
        us = graph_us(lambda: B.bi_nvfp4_quant(t["X2"], ga, Aq2, Aqs2), 50)
        point("next", "nvfp4_quant K=4096", M, us, (2.0 * M * H + M * H / 2 + M * H / 16, 0.0))
        q16, s16 = B.bi_nvfp4_quant(t["X2"][:16], ga)
        check(torch.equal(q16, Aq2[:16]) and torch.equal(s16, Aqs2[:16]), "quant rows 0..15")
        parts = [randn((M, H), 1.0, 60 + i) for i in range(8)]
        resid = randn((M, H), 1.0, 70)
        Rr, Yr = B.bi_reduce_rmsnorm(parts, t["g2"], eps, residual=resid)
        us = graph_us(lambda: B.bi_reduce_rmsnorm(parts, t["g2"], eps, resid, Rr, Yr), 50)
        point("next", "reduce 8 partials + residual, RMSNorm H=4096", M, us, (2.0 * M * H * 11 + 2.0 * H, 0.0))
        R16, Y16 = B.bi_reduce_rmsnorm([q[:16] for q in parts], t["g2"], eps, residual=resid[:16])
        check(torch.equal(R16, Rr[:16]) and torch.equal(Y16, Yr[:16]), "reduce_rmsnorm rows 0..15")
        del parts, resid, Rr, Yr
        E = 8
        sizes = np.bincount(inputs.rng(12345, 20).integers(0, E, M), minlength=E)
        offs = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int64, device=dev)
        We = randn((E, H, H), 0.02, 80)
        Ye = B.bi_grouped_gemm(t["Ao"], We, offs)
        us = graph_us(lambda: B.bi_grouped_gemm(t["Ao"], We, offs, Ye), 20)
        point("next", "grouped GEMM 8 experts x 4096x4096", M, us, (2.0 * (M * H + E * H * H + M * H), 2.0 * M * H * H),
              group_sizes=sizes.tolist())
        e0 = int(np.argmax(sizes > 0))
        r0 = int(np.sum(sizes[:e0]))
        check(torch.equal(B.bi_gemm(t["Ao"][r0:r0 + 1], We[e0]), Ye[r0:r0 + 1]), "grouped row alone")
        del We, Ye, offs
        Bq, Hq, Dqk, Dv, Lmx = 64, 16, 576, 512, 4096
        lens_np = inputs.rng(12345, 21).integers(1024, Lmx + 1, Bq).astype(np.int32)
        qa = randn((Bq, Hq, Dqk), 1.0, 90)
        kva = randn((Bq, Lmx, Dqk), 1.0, 91)
        lens_d = torch.from_numpy(lens_np).to(dev)
        wsa = torch.empty(B.mla_decode_workspace_size(Bq, Hq, Lmx, Dqk, Dv), dtype=torch.uint8, device=dev)
        sc = 1.0 / 192 ** 0.5
        oa = B.bi_mla_decode(qa, kva, lens_d, sc, Dv, workspace=wsa)
        mla_work = (2.0 * int(lens_np.sum()) * Dqk + 2.0 * Bq * Hq * (Dqk + Dv) + 4.0 * Bq,
                    2.0 * Hq * int(lens_np.sum()) * (Dqk + Dv))
        us = graph_us(lambda: B.bi_mla_decode(qa, kva, lens_d, sc, Dv, oa, workspace=wsa), 20)
        point("next", "mla_decode 64 req 1K-4K tokens, 16 heads, 576/512 (workspace)", Bq, us, mla_work)
        on = torch.empty_like(oa)
        us = graph_us(lambda: B.bi_mla_decode_noalloc(qa, kva, lens_d, sc, Dv, on), 20)
        point("next", "mla_decode, the same, no-allocation entry point", Bq, us, mla_work)
        check(torch.equal(on, oa), "mla_decode noalloc == workspace")
        o1 = B.bi_mla_decode(qa[3:4].contiguous(), kva[3:4].contiguous(), lens_d[3:4].contiguous(), sc, Dv)
        check(torch.equal(o1[0], oa[3]), "mla_decode request alone")
        check(torch.equal(B.bi_mla_decode(qa, kva, lens_d, sc, Dv), oa), "mla_decode without workspace")
        del qa, kva, oa, on, o1, wsa

        # run to run: the step's outputs are identical over repeats, eager and replayed
        for _ in range(3):
            step()
            torch.cuda.synchronize()
            for k in out:
                check(torch.equal(out[k], eager[k]), f"eager step repeat {k}")
            step_graph.replay()
            torch.cuda.synchronize()
            for k in out:
                check(torch.equal(out[k], eager[k]), f"step graph replay {k}")
        result["sweep"] = sweep

        def gmean(v):
            v = [max(x, 1e-9) for x in v]
            return float(f"{math.exp(sum(math.log(x) for x in v) / len(v)):.4g}") if v else None

        summary = {}
        for cfg in sorted({e["config"] for e in sweep}):
            es = [e for e in sweep if e["config"] == cfg and "note" not in e]
            if not es:
                continue
            summary[cfg] = {"points": len(es), "geomean_frac": gmean([e["frac"] for e in es]),
                            "min_frac": min(e["frac"] for e in es)}
            big = [e["frac"] for e in es if e["bound"] == "mfma" and e["M"] >= 2048]
            small = [e["frac"] for e in es if e["M"] <= 16 and e["bound"] == "hbm"]
            if big:
                summary[cfg]["mfma_frac_at_M_ge_2048"] = gmean(big)
            if small:
                summary[cfg]["hbm_frac_at_M_le_16"] = gmean(small)
        result["sweep_summary"] = summary
        result["fixed_plan"] = fixed
    result["invariance"] = {"checked": inv["checked"], "passed": inv["passed"],
                            "pass_pct": round(100.0 * inv["passed"] / max(1, inv["checked"]), 2),
                            "failed": inv["failed"]}

    # ---------------------------------------------------------------- oracle
    if not args.no_cpu_baseline:
        import oracle

        def oracle_rows(r):
            rows = np.arange(r)
            done = 0.0
            oracle.rmsnorm(host["X"], host["g1"], eps, rows=rows)
            for Wk, Ak, N, K in [("Wqkv", "X", Nqkv, H), ("Wo", "Ao", No, H),
                                 ("Wgu", "X2", Ngu, H), ("Wdn", "Adn", H, Kdn)]:
                oracle.gemm(host[Ak], host[Wk], rows=rows)
                done += 2.0 * r * N * K
            oracle.bmm(host["Amla"][:, :r], host["Bmla"])
            done += 2.0 * heads * r * dn * dk
            oracle.nvfp4_gemm(host["X2"], None, host["W4"], host["W4s"], alpha4, H, rows=rows)
            done += 2.0 * r * Ngu * H
            return done

        tc = time.perf_counter()
        oracle_rows(1)
        dt1 = time.perf_counter() - tc
        r = int(max(1, min(M, args.cpu_seconds / max(dt1, 1e-3))))
        log(f"oracle: 1 row {dt1:.2f}s; timing {r} rows")
        tc = time.perf_counter()
        fr = oracle_rows(r)
        dtr = time.perf_counter() - tc
        result["cpu_baseline"] = {
            "value": round(fr / dtr / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dtr, 2),
            "sample": f"first {r} of {M} rows of every GEMM-family op of the step (BMM: {r} rows per head), "
                      f"fp64 oracle, {fr / 1e9:.1f} GFLOP"}
        log(f"oracle {fr / dtr / 1e9:.2f} GFLOP/s on {oracle.num_threads()} threads")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
