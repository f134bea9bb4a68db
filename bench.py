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

Prints one JSON line.  `value` is the step's GEMM-family TFLOP/s (all flops
of the step over the measured step time).  `roofline` is for the dominant
kernel, the bf16 gate_up GEMM; its duration is measured with HIP events on
the stream it is launched on, and `traffic` comes from the committed
counter summary in profiles/ when that was taken with the current kernel
sources.  `sweep` adds per-op figures at M = 1, 16, 64, 256 and 1024 for the dense
linears (HBM GB/s and TFLOP/s with >= 1 GiB of rotating weight copies, so
the 256 MB last-level cache cannot serve them), at M = 1, 16 and 64 for the NVFP4
GEMM, and at the step's M for every op.  `invariance` counts bitwise checks of small-M
rows against the step's rows and of repeated steps.  `cpu_baseline` times
the fp64 oracle on a bounded sample of the same step.

Profiler passes (run under rocprofv3; see profiles/):
    python bench.py --only-step --calib-copy --steps 5 --warmup 2
and their summary:
    python bench.py --summarize <rocprofv3 output dir> --out <file>
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
CALIB_BYTES = 512 << 20     # bytes read (and written) by one calibration copy
GATE_UP_KERNEL = "pingpong_kernel<256>"   # bf16 GEMM, 256x256 tile, ping-pong schedule
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemm_gate_up_M2048_counters.txt")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--m", type=int, default=2048, help="tokens per step")
    p.add_argument("--no-sweep", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    p.add_argument("--only-step", action="store_true",
                   help="run the timed steps only (for profiler passes)")
    p.add_argument("--calib-copy", action="store_true",
                   help="after the steps, copy 512 MiB three times (counter calibration)")
    p.add_argument("--summarize", metavar="DIR", nargs="+",
                   help="summarise rocprofv3 CSV output in DIR(s)")
    p.add_argument("--out", metavar="FILE", help="where --summarize writes its summary")
    p.add_argument("--command", default="", help="command line recorded by --summarize")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of the HIP/C++ sources: a counter summary is valid only for them."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "invariant_deterministic_bi_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".h", ".hip", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def read_counters_summary():
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    with open(COUNTERS_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ summaries

def summarize(dirs, out, command):
    """Condense rocprofv3 CSV output (kernel stats, counters) into text.

    The gate_up GEMM's kernel instance (the 256x256 ping-pong kernel) may
    serve other GEMMs too, so its dispatches are grouped by grid size: per
    grid size the kernel trace gives the mean duration and the counters the
    mean per dispatch, and the gate_up group is the one with the largest
    FETCH_SIZE (the largest weight).  Each counter of that group is scaled by
    (true bytes of the calibration copy / what the same counter reads for
    it); traffic_bytes_per_launch is the scaled FETCH_SIZE plus the scaled
    WRITE_SIZE.
    """
    lines = [f"# rocprofv3 summary written by: python bench.py --summarize {' '.join(dirs)}",
             f"# profiled command(s): {command}" if command else "#",
             f"kernel_source_sha: {kernel_source_sha()}"]
    acc = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
            rows = list(csv.DictReader(open(path)))
            lines.append(f"# kernel stats ({os.path.basename(path)}): name | calls | avg ns | total ns | %")
            for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0) or 0)):
                lines.append(f"{r['Name'][:150]} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                             f"{float(r['TotalDurationNs']):.0f} | {float(r.get('Percentage', 0) or 0):.2f}")
        for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            groups, every = {}, {}
            for r in csv.DictReader(open(path)):
                g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
                dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                if GATE_UP_KERNEL in r["Kernel_Name"]:
                    groups.setdefault(g, []).append(dur)
                every.setdefault((r["Kernel_Name"][:110], g), []).append(dur)
            if groups:
                lines.append(f"# {GATE_UP_KERNEL} by grid size (threads): calls | avg ns")
                for g, v in sorted(groups.items()):
                    lines.append(f"grid_{g}_calls_avg_ns: {len(v)} | {sum(v) / len(v):.0f}")
            if every:
                lines.append("# every kernel by grid size (threads), largest total first: "
                             "name | grid | calls | avg ns | min ns")
                for (n, g), v in sorted(every.items(), key=lambda kv: -sum(kv[1]))[:60]:
                    lines.append(f"{n} | {g} | {len(v)} | {sum(v) / len(v):.0f} | {min(v)}")
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                name = r["Kernel_Name"]
                if GATE_UP_KERNEL in name:
                    key = ("gemm", r["Counter_Name"], int(r["Grid_Size"]))
                elif "direct_copy" in name:
                    key = ("copy", r["Counter_Name"], 0)
                else:
                    continue
                acc.setdefault(key, []).append(float(r["Counter_Value"]))
    if acc:
        mean = {k: sum(v) / len(v) for k, v in acc.items()}
        fetch = {g: m for (kind, cn, g), m in mean.items() if kind == "gemm" and cn == "FETCH_SIZE"}
        gate_grid = max(fetch, key=fetch.get) if fetch else None
        lines.append("# counters, mean per dispatch (FETCH_SIZE and WRITE_SIZE in KiB, others as read)")
        for (kind, cn, g), m in sorted(mean.items()):
            tag = f"{kind}_grid{g}" if kind == "gemm" else kind
            lines.append(f"{tag}_{cn}_per_dispatch: {m:.1f}")
            lines.append(f"{tag}_{cn}_dispatches: {len(acc[(kind, cn, g)])}")
        if gate_grid is not None:
            lines.append(f"gate_up_grid_threads: {gate_grid}")
        total, parts = 0.0, 0
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            gm, cm = mean.get(("gemm", cn, gate_grid)), mean.get(("copy", cn, 0))
            if gm is not None and cm:
                factor = CALIB_BYTES / (cm * 1024.0)
                scaled = gm * 1024.0 * factor
                lines.append(f"copy_{cn}_scale: {factor:.4f}")
                lines.append(f"gate_up_{cn}_bytes_scaled: {scaled:.0f}")
                total += scaled
                parts += 1
        if parts == 2:
            lines.append(f"traffic_bytes_per_launch: {total:.0f}")
        g = gate_grid if gate_grid is not None else (max(k[2] for k in mean if k[0] == "gemm")
                                                       if any(k[0] == "gemm" for k in mean) else None)
        lds_c, lds_a = mean.get(("gemm", "SQ_LDS_BANK_CONFLICT", g)), mean.get(("gemm", "SQ_LDS_IDX_ACTIVE", g))
        if lds_c is not None and lds_a:
            lines.append(f"gate_up_lds_bank_conflict_over_lds_active: {lds_c / lds_a:.4f}")
        mf, busy = mean.get(("gemm", "SQ_VALU_MFMA_BUSY_CYCLES", g)), mean.get(("gemm", "SQ_BUSY_CYCLES", g))
        if mf is not None and busy:
            lines.append(f"gate_up_mfma_busy_over_sq_busy: {mf / busy:.4f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.out or os.path.join(args.summarize[0], "summary.txt"),
                  args.command)
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
    flops = {
        "qkv": 2.0 * M * Nqkv * H, "bmm": 2.0 * heads * Mb * dn * dk, "o_proj": 2.0 * M * No * H,
        "gate_up": 2.0 * M * Ngu * H, "down": 2.0 * M * H * Kdn, "nvfp4_gate_up": 2.0 * M * Ngu * H,
    }
    total_flops = sum(flops.values())
    ev = []

    def step(timed=False):
        B.bi_rmsnorm(t["X"], t["g1"], eps, out["Xn"])
        B.bi_gemm(out["Xn"], t["Wqkv"], out["Yqkv"])
        B.bi_bmm(t["Amla"], t["Bmla"], out["Ymla"])
        B.bi_gemm(t["Ao"], t["Wo"], out["Yo"])
        B.bi_rmsnorm(t["X2"], t["g2"], eps, out["Xn2"])
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        B.bi_gemm(out["Xn2"], t["Wgu"], out["Ygu"])
        if timed:
            e1.record()
            ev.append((e0, e1))
        B.bi_gemm(t["Adn"], t["Wdn"], out["Ydn"])
        B.bi_nvfp4_gemm(out["Xn2"], t["W4"], t["W4s"], alpha4, out["Y4"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step(timed=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t1
    ms_per_step = elapsed * 1e3 / args.steps
    value = total_flops / (ms_per_step * 1e-3) / 1e12
    gu_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    gu_tflops = flops["gate_up"] / (gu_ms * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms, {value:.1f} TFLOP/s; gate_up {gu_ms * 1e3:.1f} us "
        f"{gu_tflops:.1f} TFLOP/s")
    if args.calib_copy:
        # a plain elementwise copy (bf16 -> fp16 conversion): reads and writes
        # exactly CALIB_BYTES each, with a kernel of its own name
        src = torch.empty(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty(CALIB_BYTES // 2, dtype=torch.float16, device=dev)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copies of {CALIB_BYTES} bytes done")
    if args.only_step:
        print(json.dumps({"metric": "step", "ms_per_step": ms_per_step, "value": value,
                          "gate_up_us": gu_ms * 1e3}), flush=True)
        return

    traffic = read_counters_summary()
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
        "roofline": {"bound": "mfma", "kernel": "bi_gemm gate_up N=24576 K=4096 (256x256 tile, ping-pong)",
                     "achieved": round(gu_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "per_launch_flops": flops["gate_up"], "avg_launch_us": round(gu_ms * 1e3, 2)},
    }

    # ---------------------------------------------------------------- sweep
    if not args.no_sweep:
        sweep = []
        inv_checked = inv_passed = 0

        def timed(fn, reps):
            fn(0)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for r in range(reps):
                fn(r)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        specs = [("qkv", t["Wqkv"], out["Xn"], out["Yqkv"], H),
                 ("o_proj", t["Wo"], t["Ao"], out["Yo"], H),
                 ("gate_up", t["Wgu"], out["Xn2"], out["Ygu"], H),
                 ("down", t["Wdn"], t["Adn"], out["Ydn"], Kdn)]
        for name, W, Afull, Yfull, K in specs:
            N = W.shape[0]
            ref = Yfull[:1024].clone()
            ncopy = max(2, int(np.ceil((1 << 30) / (W.numel() * 2))))
            copies = [W] + [W.clone() for _ in range(ncopy - 1)]
            for m in (1, 16, 64, 256, 1024):
                A = Afull[:m]
                Y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
                us = timed(lambda r: B.bi_gemm(A, copies[r % ncopy], Y), (20 if m <= 64 else 4) * ncopy)
                byt = 2.0 * (m * K + N * K + m * N)
                gbs = byt / (us * 1e-6) / 1e9
                tf = 2.0 * m * N * K / (us * 1e-6) / 1e12
                sweep.append({"op": name, "N": N, "K": K, "M": m, "us": round(us, 2),
                              "GB/s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                              "TFLOP/s": round(tf, 3), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)})
                # rows 0 .. m-1 computed with M = m equal the step's rows
                inv_checked += 1
                inv_passed += int(torch.equal(Y, ref[:m]))
            del copies
            torch.cuda.empty_cache()
        # NVFP4 gate_up at M = 1, 16 (rotating weight copies)
        ncopy = 8
        w4c = [t["W4"]] + [t["W4"].clone() for _ in range(ncopy - 1)]
        s4c = [t["W4s"]] + [t["W4s"].clone() for _ in range(ncopy - 1)]
        ref16 = out["Y4"][:64].clone()
        for m in (1, 16, 64):
            A = out["Xn2"][:m]
            Y = torch.empty((m, Ngu), dtype=torch.bfloat16, device=dev)
            us = timed(lambda r: B.bi_nvfp4_gemm(A, w4c[r % ncopy], s4c[r % ncopy], alpha4, Y), 24)
            byt = 2.0 * m * H + Ngu * H / 2 + Ngu * H / 16 + 2.0 * m * Ngu
            gbs = byt / (us * 1e-6) / 1e9
            sweep.append({"op": "nvfp4_gate_up", "N": Ngu, "K": H, "M": m, "us": round(us, 2),
                          "GB/s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
            inv_checked += 1
            inv_passed += int(torch.equal(Y, ref16[:m]))
        del w4c, s4c
        # NVFP4 activation quantiser at the step's M (K = 4096), and the W4A4
        # GEMM it feeds (gate_up weight)
        ga = inputs.nvfp4_global_scale(inputs.bf16_bits_to_f32(host["X2"]))
        Aq, Aqs = B.bi_nvfp4_quant(t["X2"], ga)
        us = timed(lambda r: B.bi_nvfp4_quant(t["X2"], ga, Aq, Aqs), 20)
        byt = 2.0 * M * H + M * H / 2 + M * H / 16
        gbs = byt / (us * 1e-6) / 1e9
        sweep.append({"op": "nvfp4_quant", "M": M, "K": H, "us": round(us, 2), "GB/s": round(gbs, 1),
                      "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
        q16, s16 = B.bi_nvfp4_quant(t["X2"][:16], ga)
        inv_checked += 1
        inv_passed += int(torch.equal(q16, Aq[:16]) and torch.equal(s16, Aqs[:16]))
        alpha44 = float(np.float32(1.0) / (ga * g4))
        Y44 = torch.empty((M, Ngu), dtype=torch.bfloat16, device=dev)
        us = timed(lambda r: B.bi_nvfp4_gemm(Aq, t["W4"], t["W4s"], alpha44, Y44, A_scales=Aqs), 10)
        tf = flops["nvfp4_gate_up"] / (us * 1e-6) / 1e12
        sweep.append({"op": "nvfp4_w4a4_gate_up", "M": M, "us": round(us, 2), "TFLOP/s": round(tf, 1),
                      "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        del Aq, Aqs, Y44
        # per-op figures at the step's M
        for name, fn, fl in [
            ("qkv", lambda r: B.bi_gemm(out["Xn"], t["Wqkv"], out["Yqkv"]), flops["qkv"]),
            ("o_proj", lambda r: B.bi_gemm(t["Ao"], t["Wo"], out["Yo"]), flops["o_proj"]),
            ("gate_up", lambda r: B.bi_gemm(out["Xn2"], t["Wgu"], out["Ygu"]), flops["gate_up"]),
            ("down", lambda r: B.bi_gemm(t["Adn"], t["Wdn"], out["Ydn"]), flops["down"]),
            ("nvfp4_gate_up", lambda r: B.bi_nvfp4_gemm(out["Xn2"], t["W4"], t["W4s"], alpha4, out["Y4"]),
             flops["nvfp4_gate_up"]),
            ("bmm", lambda r: B.bi_bmm(t["Amla"], t["Bmla"], out["Ymla"]), flops["bmm"]),
        ]:
            us = timed(fn, 10)
            tf = fl / (us * 1e-6) / 1e12
            sweep.append({"op": name, "M": M if name != "bmm" else Mb, "us": round(us, 2),
                          "TFLOP/s": round(tf, 1), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        us = timed(lambda r: B.bi_rmsnorm(t["X"], t["g1"], eps, out["Xn"]), 20)
        gbs = (4.0 * M * H + 2.0 * H) / (us * 1e-6) / 1e9
        sweep.append({"op": "rmsnorm", "M": M, "H": H, "us": round(us, 2), "GB/s": round(gbs, 1),
                      "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
        # grouped (mixture-of-experts) GEMM: the step's M tokens routed to 8
        # experts of [4096, 4096] with seeded, uneven group sizes
        E = 8
        sizes = np.bincount(inputs.rng(12345, 20).integers(0, E, M), minlength=E)
        offs = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int64, device=dev)
        We = torch.randn((E, H, H), device=dev).mul_(0.02).to(torch.bfloat16)
        Ye = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        us = timed(lambda r: B.bi_grouped_gemm(t["Ao"], We, offs, Ye), 10)
        tf = 2.0 * M * H * H / (us * 1e-6) / 1e12
        sweep.append({"op": "grouped_gemm_8x4096x4096", "M": M, "group_sizes": sizes.tolist(),
                      "us": round(us, 2), "TFLOP/s": round(tf, 1), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        e0 = int(np.argmax(sizes > 0))
        t0 = int(np.sum(sizes[:e0]))
        inv_checked += 1
        inv_passed += int(torch.equal(B.bi_gemm(t["Ao"][t0:t0 + 1], We[e0]), Ye[t0:t0 + 1]))
        del We, Ye, offs
        # fixed-order reduction of 8 per-rank partial outputs (a row-parallel
        # layer's [M, 4096] at tensor-parallel degree 8) + residual, then RMSNorm
        parts = [torch.randn((M, H), device=dev).to(torch.bfloat16) for _ in range(8)]
        resid = torch.randn((M, H), device=dev).to(torch.bfloat16)
        Rr, Yr = B.bi_reduce_rmsnorm(parts, t["g2"], eps, residual=resid)
        us = timed(lambda r: B.bi_reduce_rmsnorm(parts, t["g2"], eps, resid, Rr, Yr), 20)
        byt = 2.0 * M * H * (len(parts) + 3) + 2.0 * H
        gbs = byt / (us * 1e-6) / 1e9
        sweep.append({"op": "reduce8_rmsnorm", "M": M, "H": H, "us": round(us, 2), "GB/s": round(gbs, 1),
                      "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
        R16, Y16 = B.bi_reduce_rmsnorm([q[:16] for q in parts], t["g2"], eps, residual=resid[:16])
        inv_checked += 1
        inv_passed += int(torch.equal(R16, Rr[:16]) and torch.equal(Y16, Yr[:16]))
        del parts, resid, Rr, Yr
        # decode attention over a latent cache: 64 requests of 1024..4096
        # tokens (seeded), 16 heads, Dqk 576 (512 latent + 64 rotary), Dv 512
        Bq, Hq, Dqk, Dv, Lmx = 64, 16, 576, 512, 4096
        lens_np = inputs.rng(12345, 21).integers(1024, Lmx + 1, Bq).astype(np.int32)
        qa = torch.randn((Bq, Hq, Dqk), device=dev).to(torch.bfloat16)
        kva = torch.randn((Bq, Lmx, Dqk), device=dev).to(torch.bfloat16)
        lens_d = torch.from_numpy(lens_np).to(dev)
        wsa = torch.empty(B.mla_decode_workspace_size(Bq, Hq, Lmx, Dqk, Dv), dtype=torch.uint8, device=dev)
        oa = B.bi_mla_decode(qa, kva, lens_d, 1.0 / 192 ** 0.5, Dv, workspace=wsa)
        us = timed(lambda r: B.bi_mla_decode(qa, kva, lens_d, 1.0 / 192 ** 0.5, Dv, oa, workspace=wsa), 10)
        byt = 2.0 * int(lens_np.sum()) * Dqk + 2.0 * Bq * Hq * (Dqk + Dv) + 4.0 * Bq
        gbs = byt / (us * 1e-6) / 1e9
        sweep.append({"op": "mla_decode", "schedule": "workgroup per 1024-token chunk + fold", "B": Bq, "H": Hq, "Dqk": Dqk, "Dv": Dv,
                      "tokens": int(lens_np.sum()), "us": round(us, 2), "GB/s": round(gbs, 1),
                      "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)})
        o1 = B.bi_mla_decode(qa[3:4].contiguous(), kva[3:4].contiguous(), lens_d[3:4].contiguous(),
                             1.0 / 192 ** 0.5, Dv)
        inv_checked += 2
        inv_passed += int(torch.equal(o1[0], oa[3]))
        inv_passed += int(torch.equal(B.bi_mla_decode(qa, kva, lens_d, 1.0 / 192 ** 0.5, Dv), oa))
        del qa, kva, oa, o1, wsa
        # run-to-run: the step's outputs are identical over repeats
        snap = {k: v.clone() for k, v in out.items()}
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        for k in out:
            inv_checked += 1
            inv_passed += int(torch.equal(out[k], snap[k]))
        result["sweep"] = sweep
        result["invariance"] = {"checked": inv_checked, "passed": inv_passed,
                                "pass_pct": round(100.0 * inv_passed / max(1, inv_checked), 2)}

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
            "sample": f"first {r} of {M} rows of every op of the step (BMM: {r} rows per head), "
                      f"fp64 oracle, {fr / 1e9:.1f} GFLOP"}
        log(f"oracle {fr / dtr / 1e9:.2f} GFLOP/s on {oracle.num_threads()} threads")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
