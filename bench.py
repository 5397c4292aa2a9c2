"""Throughput of the weight-only-int4 GEMM path on one MI355X.

A step is one W4A8 call on the decode-batch workload (M = 64 tokens, one per
concurrent sequence; K = N = 5120; int4 group-128 weights with signed fp16
scales): per-token int8 quantisation of the activations, then the int8
matrix-core GEMM with per-group rescale.  Inputs are seeded synthetic tensors
already resident in HBM.  The weights rotate over enough packed copies that
every call reads a copy not touched for > 512 MB of traffic, so the 256 MB
Infinity Cache cannot serve repeats.  Steps are captured in a HIP graph and
replayed; the timed region is bracketed by device synchronisation.

Printed: one JSON line.  `value` is algorithmic HBM bytes per step (weights,
scales, fp16 activations, fp16 output, each counted once) per second.
`roofline` is the dominant kernel (the GEMM, timed alone via
w4a8_gemm_prepared) against the 8 TB/s HBM peak.  `cpu_baseline` is the
numpy oracle on the same workload on the host's cores.  `per_workload` adds
the verify (W4A16, M = 8/16, N = 34816), prefill (W4A8, M = 4096, K = 17408)
and vocabulary (int8 gather + lm_head over 248,320 rows) workloads measured
the same way, for information, and two lm_head variants: a 40,960-row draft
head gathered from the int8 table (M = 1) and an int4 head over all 248,320
rows (W4A16, M = 16 and 64); the RMSNorm fused with the W4A8 quantiser at
the decode and prefill shapes; and the split-KV verify attention (one layer,
5 query tokens, 1.5k and 16k context).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A8/W4A16 GEMM TOPS + HBM GB/s (% roofline) at M=8/64/4096, K=N=5120"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
FP16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the per-workload extras")
    ap.add_argument("--extras", default=",".join(EXTRA_SECTIONS),
                    help="comma list of the per-workload sections to run: " + ", ".join(EXTRA_SECTIONS))
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip the amd-smi clock reading (also skipped under rocprofv3, whose preloaded "
                         "library would follow amd-smi into its child process)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 1 GiB device copy that calibrates the FETCH_SIZE / WRITE_SIZE "
                         "counters (run it under rocprofv3 --pmc), then exit")
    ap.add_argument("--floor", action="store_true",
                    help="only time the load floors of the decode GEMM's operand walk (qg_probe_read: "
                         "a plain read of its weights, its own access pattern, an empty launch), then exit")
    ap.add_argument("--vendor", action="store_true",
                    help="only time the vendor library's plain GEMMs (hipBLASLt through torch: int8, fp8, "
                         "bf16) at the prefill shape beside this library's W4A8 GEMM, then exit")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of 1 GiB whose source is out of the caches
    (filled, then a second 1 GiB buffer filled), three times, so that the
    traffic counters can be scaled against bytes known to move."""
    import torch
    n = 1 << 30
    dev = torch.device("cuda:0")
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    c = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    c.fill_(2)
    for _ in range(3):
        b.copy_(a)
        c.fill_(3)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}))


def load_floor():
    """Per-launch times, in a replayed graph, of reads with the decode GEMM's
    operand walk and none of its arithmetic (qg_probe_read): its packed
    weights (13,107,200 B, rotated over copies past the Infinity Cache) read
    as 256 contiguous slices, then as the row split reads them (128 n-block
    slices, each read by its two m-groups on one XCD, plus each m-group's
    half of the 327,680 B of codes), the same with four m-groups per slice
    (the split of 16-row m-groups over blocks of 5 n-tiles), and a launch of
    that grid that reads nothing."""
    import torch
    import spec_verify_amd as qg
    import synth
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS["decode_w4a8"]
    K, N = cfg["K"], cfg["N"]
    wbytes = N * K // 2
    n = copies_for(wbytes)
    w = [torch.full((wbytes,), 3, dtype=torch.uint8, device=dev) for _ in range(n)]
    codes = torch.full((cfg["M"] * K,), 5, dtype=torch.uint8, device=dev)
    none = torch.empty((0,), dtype=torch.uint8, device=dev)
    sink = torch.empty((256 * 640 // 64,), dtype=torch.int32, device=dev)
    cases = {
        "empty_launch_256x512": lambda i: qg.qg_probe_read(none, None, 1, 256, 512, True, sink),
        "plain_weights_256x640": lambda i: qg.qg_probe_read(w[i % n], None, 1, 256, 640, True, sink),
        "decode_walk_weights_256x512": lambda i: qg.qg_probe_read(w[i % n], None, 2, 256, 512, True, sink),
        "decode_walk_256x512": lambda i: qg.qg_probe_read(w[i % n], codes, 2, 256, 512, True, sink),
        "decode_walk_hot_256x512": lambda i: qg.qg_probe_read(w[0], codes, 2, 256, 512, True, sink),
        "share4_walk_weights_256x512": lambda i: qg.qg_probe_read(w[i % n], None, 4, 256, 512, True, sink),
        "share4_walk_256x512": lambda i: qg.qg_probe_read(w[i % n], codes, 4, 256, 512, True, sink),
    }
    out = {}
    for name, fn in cases.items():
        us, _ = graph_time_us(torch, fn, 200, reps=3)
        out[name] = round(us, 3)
        print(f"# floor: {name} {out[name]} us", file=sys.stderr, flush=True)
    print(json.dumps({"load_floor_us_per_launch": out, "weight_bytes": wbytes, "code_bytes": cfg["M"] * K,
                      "weight_copies": n}))


def vendor_reference():
    """The vendor library's dense GEMMs at the prefill shape (M = 4096,
    K = 17408, N = 5120), as context for the W4A8 kernel's matrix-core
    fraction: torch._int_mm (int8 x int8 -> int32), torch._scaled_mm (fp8
    e4m3, unit scales, fp16 out) and torch.mm (bf16), each hipBLASLt, with
    the weight operand [N, K] read transposed and rotated over copies past
    the Infinity Cache, timed eagerly with HIP events (about 0.4 ms per
    call, so launch gaps do not count), best of three runs.  Beside them,
    this library's w4a8_gemm_prepared (the GEMM alone on prepared codes)
    and w4a8_gemm (quantiser + GEMM), timed the same way.  The vendor GEMMs
    do no int4 unpack and no per-group rescale."""
    import torch
    import spec_verify_amd as qg
    import synth
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS["prefill_w4a8"]
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    ops = 2.0 * M * N * K
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def eager_us(fn, n_calls, reps=3):
        best = float("inf")
        for _ in range(reps):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(n_calls):
                fn(i)
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b) * 1e3 / n_calls)
        return best

    out = {}

    def entry(name, fn, n, ncopy, peak):
        us = eager_us(fn, 4 * n)
        out[name] = dict(us_per_call=round(us, 2), TOPS=round(ops / us / 1e6, 1),
                         frac_peak=round(ops / us / 1e6 / peak, 4), weight_copies=ncopy)
        print(f"# vendor: {name} {out[name]}", file=sys.stderr, flush=True)

    a8 = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=gen)
    n8 = copies_for(N * K)
    b8 = [torch.randint(-8, 8, (N, K), dtype=torch.int8, device=dev, generator=gen) for _ in range(n8)]
    entry("int8_int_mm_hipblaslt", lambda i: torch._int_mm(a8, b8[i % n8].t()), n8, n8, INT8_PEAK_TOPS)
    del b8
    fp8 = getattr(torch, "float8_e4m3fn")
    af = torch.randn((M, K), dtype=torch.float16, device=dev, generator=gen).to(fp8)
    bf = [torch.randn((N, K), dtype=torch.float16, device=dev, generator=gen).to(fp8) for _ in range(n8)]
    one = torch.ones((), dtype=torch.float32, device=dev)
    entry("fp8_e4m3_scaled_mm_hipblaslt",
          lambda i: torch._scaled_mm(af, bf[i % n8].t(), scale_a=one, scale_b=one, out_dtype=torch.float16),
          n8, n8, INT8_PEAK_TOPS)
    del af, bf
    ab = torch.randn((M, K), dtype=torch.bfloat16, device=dev, generator=gen)
    n16 = copies_for(N * K * 2)
    bb = [torch.randn((N, K), dtype=torch.bfloat16, device=dev, generator=gen) for _ in range(n16)]
    entry("bf16_mm_hipblaslt", lambda i: torch.mm(ab, bb[i % n16].t()), n16, n16, FP16_PEAK_TFLOPS)
    del ab, bb
    torch.cuda.empty_cache()

    x, codes, scales = synth.gemm_inputs(cfg)
    xd = torch.from_numpy(x).to(dev)
    wp, sp = qg.w4_repack(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
    nw = copies_for(wp.numel() + sp.numel() * 2)
    copies = [(wp, sp)] + [(wp.clone(), sp.clone()) for _ in range(nw - 1)]
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    prep = qg.w4a8_prepare(xd)
    entry("w4a8_gemm_prepared", lambda i: qg.w4a8_gemm_prepared(prep, M, K, copies[i % nw][0], copies[i % nw][1],
                                                                 N, y=y), nw, nw, INT8_PEAK_TOPS)
    ws = torch.empty((qg.qg_workspace_bytes(qg.QG_OP_W4A8, M, K, N),), dtype=torch.uint8, device=dev)
    entry("w4a8_gemm", lambda i: qg.w4a8_gemm(xd, copies[i % nw][0], copies[i % nw][1], N, y=y, workspace=ws),
          nw, nw, INT8_PEAK_TOPS)
    print(json.dumps({"vendor_reference": out, "M": M, "K": K, "N": N}))


def gemm_bytes(M, K, N):
    """Algorithmic HBM bytes of one W4A*/W4A16 GEMM call: packed int4 weights,
    fp16 group scales, fp16 activations, fp16 output."""
    return N * K // 2 + N * (K // 128) * 2 + M * K * 2 + M * N * 2


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_w4a8_m64_k5120_n5120_traffic.md")
KERNEL_SOURCES = ["spec_verify_amd/csrc/gemm_skinny.hip", "spec_verify_amd/csrc/operands.h",
                  "spec_verify_amd/csrc/common.h"]


def measured_traffic():
    """HBM bytes per launch of the decode GEMM from the committed counter
    passes (FETCH_SIZE and WRITE_SIZE, calibrated), or None when the kernel's
    sources have changed since they were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
        h = hashlib.sha256()
        for f in KERNEL_SOURCES:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and
                      line.split(": ", 1)[0] in ("traffic_bytes_per_launch", "kernel_sources_sha256"))
        if fields["kernel_sources_sha256"].split()[0] != h.hexdigest():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copies_for(nbytes):
    return max(2, -(-2 * MALL_BYTES // nbytes) + 1)


def graph_time_us(torch, fn, n_calls, reps=1):
    """Capture n_calls of fn(i) in a graph, replay it for about 50 ms to
    warm, then time at least `reps` replays and at least 20 ms of them;
    return microseconds per call (HIP events on the replay stream)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_calls):
            fn(i)
    # Warm for about 50 ms of back-to-back replays, then time at least
    # 20 ms of them: after the idle capture the part takes some milliseconds
    # to settle (per pair of replays, prefill read 428, 399, then 390-396
    # us per call; verify at M = 8 18.3, then 21-23 us for about 10 ms,
    # then 17.8-18.6 us), and a replay of a few calls alone varies by a few
    # percent.  The decode graphs read the same either way.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    replay_us = max(e0.elapsed_time(e1) * 1e3, 1.0)
    for _ in range(min(2000, max(2, int(50e3 / replay_us)))):
        g.replay()
    torch.cuda.synchronize()
    reps = max(reps, min(2000, int(20e3 / replay_us)))
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (n_calls * reps), g


def clocks_under_load(torch, graph, replays, tries=1):
    """Clocks and socket power read with amd-smi while `graph` replays
    (`replays` times, enqueued before the query so the GPU is busy while it
    runs).  With tries > 1 the whole sequence repeats and the reading with
    the highest socket power is kept (a reading sometimes lands after the
    replays have drained).  None when amd-smi is missing or fails; the bench
    never depends on it."""
    import shutil
    smi = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if smi is None:
        return None
    best = None
    for _ in range(tries):
        r = _clock_reading(torch, graph, replays, smi)
        if r is not None and (best is None or (r["socket_power_w"] or 0) > (best["socket_power_w"] or 0)):
            best = r
    return best


def _clock_reading(torch, graph, replays, smi):
    import subprocess
    for _ in range(replays):
        graph.replay()
    try:
        r = subprocess.run([smi, "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True, text=True,
                           timeout=30)
        torch.cuda.synchronize()
        d = json.loads(r.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clk = g["clock"]
        gfx = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
        mem = [v["clk"]["value"] for k, v in clk.items() if k.startswith("mem_") and isinstance(v.get("clk"), dict)]
        gmax = [v["max_clk"]["value"] for k, v in clk.items() if k.startswith("gfx_") and isinstance(v.get("max_clk"), dict)]
        pw = g.get("power", {}).get("socket_power", {})
        return dict(source="amd-smi metric -c -p during graph replay", gfx_mhz=gfx, gfx_max_mhz=max(gmax) if gmax else None,
                    mem_mhz=mem, socket_power_w=pw.get("value") if isinstance(pw, dict) else None)
    except Exception:  # noqa: BLE001 -- reporting only
        torch.cuda.synchronize()
        return None


def cpu_baseline(x, codes, scales, seconds):
    """The numpy oracle (quantise, exact group partials, float64 rescale) on the
    decode workload, repeated for about `seconds` on the host's cores."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    M, K = x.shape
    N = codes.shape[0]
    with threadpool_limits(limits=os.cpu_count() or 1):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        oracle.ref_w4a8(x, codes, scales)     # warm up
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.ref_w4a8(x, codes, scales)
            n += 1
            dt = time.perf_counter() - t0
            if dt >= seconds:
                break
    per_call = dt / n
    return dict(value=round(gemm_bytes(M, K, N) / per_call / 1e9, 3), unit="GB/s", cores=int(threads),
                kind="oracle", seconds_per_call=round(per_call, 5),
                sample=f"{n} full oracle evaluations of the decode workload (M=64, K=N=5120) in {dt:.1f} s")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the path is single-GPU and no multi-GPU run is defined "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.floor:
        load_floor()
        return
    if args.vendor:
        vendor_reference()
        return

    import numpy as np
    import torch

    import spec_verify_amd as qg
    import synth

    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS["decode_w4a8"]
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    x, codes, scales = synth.gemm_inputs(cfg)
    xd = torch.from_numpy(x).to(dev)
    wp, sp = qg.w4_repack(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
    ncopy = copies_for(wp.numel() + sp.numel() * 2)
    copies = [(wp.clone(), sp.clone()) for _ in range(ncopy)]
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    ws = torch.empty((qg.qg_workspace_bytes(qg.QG_OP_W4A8, M, K, N),), dtype=torch.uint8, device=dev)

    def step(i):
        w, s = copies[i % ncopy]
        qg.w4a8_gemm(xd, w, s, N, y=y, workspace=ws)

    # warmup graph, then the timed graph of exactly `steps` calls
    graph_time_us(torch, step, max(1, args.warmup))
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(args.steps):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / args.steps
    step_bytes = gemm_bytes(M, K, N)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # dominant kernel: the GEMM alone on prepared (quantised) activations
    prep = qg.w4a8_prepare(xd)
    torch.cuda.synchronize()
    gemm_us, _ = graph_time_us(
        torch, lambda i: qg.w4a8_gemm_prepared(prep, M, K, copies[i % ncopy][0], copies[i % ncopy][1], N, y=y),
        max(ncopy, 200))
    kernel_bytes = N * K // 2 + N * (K // 128) * 2 + M * K + M * 4 + M * N * 2
    achieved = kernel_bytes / (gemm_us * 1e-6) / 1e9
    roofline = dict(bound="hbm", kernel="skinny_kernel<W4A8, 3 n-tiles, 2 m-tiles, 8 waves, ring 1> (n-blocks of 2 or 3 tiles, rows split over 2 workgroups, w4a8_gemm_prepared)", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                    bytes_per_launch=kernel_bytes, avg_launch_us=round(gemm_us, 3), traffic=measured_traffic())

    out = dict(metric=METRIC, value=round(value, 2), unit="GB/s", n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=round(ms_per_step, 6), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="int8", data="synthetic",
               config=dict(workload="decode_w4a8: W4A8 GEMM, M=64 tokens, K=5120, N=5120, int4 group-128 "
                                    "weights with signed fp16 scales, fp16 activations N(0,1) with 1% x20 "
                                    "outliers, quantised per token inside the call, fp16 output",
                           M=M, K=K, N=N, weight_copies=ncopy, graph_replay=True),
               tops=round(2 * M * N * K / (ms_per_step * 1e-3) / 1e12, 3),
               frac_hbm=round(value / HBM_PEAK_GBS, 4), wall_s=round(wall, 4), roofline=roofline)

    # SCLK / MCLK and socket power while the timed graph replays (about three
    # seconds of replays are queued, so the GPU is still busy when amd-smi,
    # which takes a second or more to start, reads them)
    under_profiler = any(k.startswith("ROCPROF") for k in os.environ)
    out["clocks"] = (None if args.no_clocks or under_profiler
                     else clocks_under_load(torch, g, max(1, int(3.0 / max(ms * 1e-3, 1e-6)))))

    if not args.no_extra:
        out["per_workload"] = extras(torch, qg, synth, np, dev, set(args.extras.split(",")),
                                     clocks=not (args.no_clocks or under_profiler))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, codes, scales, args.cpu_seconds)
    print(json.dumps(out), flush=True)


EXTRA_SECTIONS = ("gemm", "norm", "attention", "vocab", "heads", "sampler")


def extras(torch, qg, synth, np, dev, sections, clocks=False):
    res = {}

    def done(section):
        print(f"# bench: {section} measured", file=sys.stderr, flush=True)

    for name in (("verify_w4a16_m8", "verify_w4a16_m16", "prefill_w4a8") if "gemm" in sections else ()):
        cfg = synth.CONFIGS[name]
        M, K, N = cfg["M"], cfg["K"], cfg["N"]
        x, codes, scales = synth.gemm_inputs(cfg)
        xd = torch.from_numpy(x).to(dev)
        wp, sp = qg.w4_repack(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
        ncopy = copies_for(wp.numel() + sp.numel() * 2)
        copies = [(wp, sp)] + [(wp.clone(), sp.clone()) for _ in range(ncopy - 1)]
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        if cfg["op"] == "w4a8":
            ws = torch.empty((qg.qg_workspace_bytes(qg.QG_OP_W4A8, M, K, N),), dtype=torch.uint8, device=dev)
            fn = lambda i: qg.w4a8_gemm(xd, copies[i % ncopy][0], copies[i % ncopy][1], N, y=y, workspace=ws)
        else:
            fn = lambda i: qg.w4a16_gemm(xd, copies[i % ncopy][0], copies[i % ncopy][1], N, y=y)
        n_calls = 4 * ncopy if M <= 64 else ncopy
        us, gg = graph_time_us(torch, fn, n_calls, reps=2)
        b = gemm_bytes(M, K, N)
        ops = 2 * M * N * K
        peak_ops = INT8_PEAK_TOPS if cfg["op"] == "w4a8" else FP16_PEAK_TFLOPS
        res[name] = dict(M=M, K=K, N=N, us_per_call=round(us, 3), GBps=round(b / us / 1e3, 1),
                         frac_hbm=round(b / us / 1e3 / HBM_PEAK_GBS, 4), TOPS=round(ops / us / 1e6, 2),
                         frac_mfma=round(ops / us / 1e6 / peak_ops, 4), weight_copies=ncopy)
        if cfg["op"] == "w4a8" and M > 64:
            # the GEMM alone, on activations quantised once beforehand
            prep = qg.w4a8_prepare(xd)
            gus, _ = graph_time_us(torch, lambda i: qg.w4a8_gemm_prepared(prep, M, K, copies[i % ncopy][0],
                                                                          copies[i % ncopy][1], N, y=y),
                                   n_calls, reps=2)
            res[name]["gemm_only"] = dict(us_per_call=round(gus, 3), TOPS=round(ops / gus / 1e6, 2),
                                          frac_mfma=round(ops / gus / 1e6 / peak_ops, 4))
            del prep
        if clocks and M > 64:
            # the matrix-core workload: does the part hold its clock under it?
            res[name]["clocks"] = clocks_under_load(torch, gg, max(1, int(3.0 / (us * n_calls * 1e-6))), tries=3)
        del copies, wp, sp
        torch.cuda.empty_cache()
        done(name)

    # the quantiser fused into the norm that makes its input (one launch per
    # hidden state; the prepared buffer then feeds every W4A8 GEMM of it)
    for name in (("decode_w4a8", "prefill_w4a8") if "norm" in sections else ()):
        cfg = synth.CONFIGS[name]
        M, H = cfg["M"], cfg["K"]
        x = torch.from_numpy(synth.acts(M, H, cfg["sigma"], cfg["p"], cfg["factor"], cfg["seed"] + 100)).to(dev)
        wn = torch.from_numpy(synth.acts(1, H, 0.1, 0.0, 1.0, cfg["seed"] + 400)[0]).to(dev)
        prep = torch.empty((qg.w4a8_prepared_bytes(M, H),), dtype=torch.uint8, device=dev)
        yn = torch.empty((M, H), dtype=torch.float16, device=dev)
        us, _ = graph_time_us(torch, lambda i: qg.rmsnorm_w4a8_prepare(x, wn, 1e-6, prepared=prep, y=yn), 20, reps=5)
        b = M * H * 2 + H * 2 + M * H * 2 + M * H + M * 4      # x, w in; y, codes, token scales out
        res[f"rmsnorm_w4a8_prepare_m{M}"] = dict(M=M, H=H, us_per_call=round(us, 3), GBps=round(b / us / 1e3, 1),
                                                 frac_hbm=round(b / us / 1e3 / HBM_PEAK_GBS, 4))
        del x, prep, yn
        done(f"rmsnorm_w4a8_prepare_m{M}")

    # split-KV verify attention, one layer: 5 query tokens (1 + 4 drafts), 24
    # query heads over 4 key/value heads, head_dim 256, 1.5k and 16k context;
    # caches rotated so that the Infinity Cache cannot serve repeats
    acfg = synth.CONFIGS["verify_attention"]
    T, Hq, Hkv = acfg["T"], acfg["Hq"], acfg["Hkv"]
    for L in (acfg["L"] if "attention" in sections else ()):
        q, kc, vc = synth.attention_inputs(T, Hq, Hkv, L, acfg["seed"])
        qd = torch.from_numpy(q).to(dev)
        kd, vd = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
        ncopy = copies_for(kd.numel() * 4)
        caches = [(kd, vd)] + [(kd.clone(), vd.clone()) for _ in range(ncopy - 1)]
        o = torch.empty((T, Hq, 256), dtype=torch.float16, device=dev)
        ws = torch.empty((qg.verify_attention_workspace_bytes(T, Hq, Hkv, L),), dtype=torch.uint8, device=dev)
        us, _ = graph_time_us(torch, lambda i: qg.verify_attention_f16(qd, caches[i % ncopy][0], caches[i % ncopy][1],
                                                                      o=o, workspace=ws), 2 * ncopy, reps=2)
        b = 2 * L * Hkv * 256 * 2 + 2 * T * Hq * 256 * 2      # keys and values once, queries and outputs
        res[f"verify_attention_t{T}_l{L}"] = dict(T=T, Hq=Hq, Hkv=Hkv, L=L, us_per_call=round(us, 3),
                                                  GBps=round(b / us / 1e3, 1),
                                                  frac_hbm=round(b / us / 1e3 / HBM_PEAK_GBS, 4), cache_copies=ncopy)
        del caches, kd, vd, ws
        torch.cuda.empty_cache()
        done(f"verify_attention_t{T}_l{L}")
    if not sections & {"vocab", "heads", "sampler"}:
        return res

    cfg = synth.CONFIGS["vocab_int8"]
    V, H = cfg["V"], cfg["H"]
    if sections & {"vocab", "heads"}:
        src = torch.from_numpy(synth.table_source(V, H, cfg["seed"] + 200).view(np.int16)).to(dev)
        Q, S = qg.quant_table_int8(src)
        del src
    if "vocab" in sections:
        ids = torch.from_numpy(synth.token_ids(cfg["T"], V, cfg["seed"] + 300)).to(dev)
        out = torch.empty((cfg["T"], H), dtype=torch.float16, device=dev)
        us, _ = graph_time_us(torch, lambda i: qg.embed_gather_dequant_int8(ids, Q, S, out=out), 200)
        res["vocab_gather_t64"] = dict(T=cfg["T"], H=H, us_per_call=round(us, 3),
                                       bytes=cfg["T"] * (H + H // 128 * 2 + H * 2))
        x = torch.from_numpy(synth.acts(cfg["M"], H, cfg["sigma"], cfg["p"], cfg["factor"], cfg["seed"] + 100)).to(dev)
        y = torch.empty((cfg["M"], V), dtype=torch.float16, device=dev)
        us, _ = graph_time_us(torch, lambda i: qg.w8a16_gemm(x, Q, S, y=y), 10, reps=2)
        b = V * H + V * (H // 128) * 2 + cfg["M"] * H * 2 + cfg["M"] * V * 2
        res["lm_head_w8a16_m64"] = dict(M=cfg["M"], K=H, N=V, us_per_call=round(us, 3), GBps=round(b / us / 1e3, 1),
                                        frac_hbm=round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                                        TFLOPS=round(2 * cfg["M"] * V * H / us / 1e6, 2))
        del y
        done("vocab_gather_t64, lm_head_w8a16_m64")
    if "heads" in sections:
        res.update(head_variants(torch, qg, synth, dev, Q, S, V, H))
    if sections & {"vocab", "heads"}:
        del Q, S
        torch.cuda.empty_cache()
    if "sampler" in sections:
        res.update(sampler_rows(torch, qg, synth, dev))
    return res


def head_variants(torch, qg, synth, dev, Q, S, V, H):
    res = {}

    # lm_head variants: the 40,960-row draft head gathered once from the same
    # table (copies rotated: 210 MB would otherwise stay in the Infinity Cache)
    dcfg = synth.CONFIGS["draft_head_int8"]
    D, Md = dcfg["D"], dcfg["M"]
    dids = torch.from_numpy(synth.draft_ids(D, V, dcfg["seed"])).to(dev)
    DQ, DS = Q.index_select(0, dids).contiguous(), S.index_select(0, dids).contiguous()
    ncopy = copies_for(DQ.numel() + DS.numel() * 2)
    dcopies = [(DQ, DS)] + [(DQ.clone(), DS.clone()) for _ in range(ncopy - 1)]
    xd = torch.from_numpy(synth.acts(Md, H, dcfg["sigma"], dcfg["p"], dcfg["factor"], dcfg["seed"] + 100)).to(dev)
    yd = torch.empty((Md, D), dtype=torch.float16, device=dev)
    us, _ = graph_time_us(torch, lambda i: qg.w8a16_gemm(xd, dcopies[i % ncopy][0], dcopies[i % ncopy][1], y=yd),
                          4 * ncopy, reps=2)
    b = D * H + D * (H // 128) * 2 + Md * H * 2 + Md * D * 2
    res["draft_head_w8a16_m1"] = dict(M=Md, K=H, N=D, us_per_call=round(us, 3), GBps=round(b / us / 1e3, 1),
                                      frac_hbm=round(b / us / 1e3 / HBM_PEAK_GBS, 4), weight_copies=ncopy)
    del dcopies, DQ, DS
    torch.cuda.empty_cache()
    print("# bench: draft_head_w8a16_m1 measured", file=sys.stderr, flush=True)

    # ... and an int4 head (W4A16 over all 248,320 rows), at verify and batch M
    wcfg = synth.CONFIGS["lm_head_w4a16"]
    K, N = wcfg["K"], wcfg["N"]
    codes, scales = synth.weights(N, K, wcfg["seed"])
    wp, sp = qg.w4_repack(torch.from_numpy(codes).to(dev), torch.from_numpy(scales).to(dev))
    del codes, scales
    ncopy = copies_for(wp.numel() + sp.numel() * 2)
    wcopies = [(wp, sp)] + [(wp.clone(), sp.clone()) for _ in range(ncopy - 1)]
    for M in (16, wcfg["M"]):
        xw = torch.from_numpy(synth.acts(M, K, wcfg["sigma"], wcfg["p"], wcfg["factor"], wcfg["seed"] + 100)).to(dev)
        yw = torch.empty((M, N), dtype=torch.float16, device=dev)
        us, _ = graph_time_us(torch, lambda i: qg.w4a16_gemm(xw, wcopies[i % ncopy][0], wcopies[i % ncopy][1], N,
                                                             y=yw), 2 * ncopy, reps=2)
        b = gemm_bytes(M, K, N)
        res[f"lm_head_w4a16_m{M}"] = dict(M=M, K=K, N=N, us_per_call=round(us, 3), GBps=round(b / us / 1e3, 1),
                                          frac_hbm=round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                                          TFLOPS=round(2 * M * N * K / us / 1e6, 2), weight_copies=ncopy)
        print(f"# bench: lm_head_w4a16_m{M} measured", file=sys.stderr, flush=True)
    del wcopies, wp, sp
    torch.cuda.empty_cache()
    return res


def sampler_rows(torch, qg, synth, dev):
    res = {}
    # top-k / top-p sampler over the logit rows (copies rotated past the
    # Infinity Cache); bytes: the logits once, the outputs
    scfg = synth.CONFIGS["sampler"]
    V, k = scfg["V"], scfg["k"]
    for R in scfg["R"]:
        xs, us_ = synth.sampler_inputs(R, V, scfg["seed"])
        xs_d = torch.from_numpy(xs).to(dev)
        ud = torch.from_numpy(us_).to(dev)
        ncopy = copies_for(xs_d.numel() * 2)
        lcopies = [xs_d] + [xs_d.clone() for _ in range(ncopy - 1)]
        outs = (torch.empty((R, k), dtype=torch.int32, device=dev), torch.empty((R, k), dtype=torch.float32, device=dev),
                torch.empty((R,), dtype=torch.int32, device=dev), torch.empty((R,), dtype=torch.int32, device=dev),
                torch.empty((R,), dtype=torch.float32, device=dev))
        ws = torch.empty((qg.sampler_workspace_bytes(R, V, k),), dtype=torch.uint8, device=dev)
        us, _ = graph_time_us(torch, lambda i: qg.sample_topk_topp(lcopies[i % ncopy], ud, k, scfg["top_p"], scfg["T"],
                                                                   out=outs, workspace=ws), 2 * ncopy, reps=2)
        b = R * V * 2 + R * (k * 8 + 12)
        res[f"sampler_r{R}_v{V}_k{k}"] = dict(R=R, V=V, k=k, top_p=scfg["top_p"], T=scfg["T"], us_per_call=round(us, 3),
                                             us_per_row=round(us / R, 3), GBps=round(b / us / 1e3, 1),
                                             frac_hbm=round(b / us / 1e3 / HBM_PEAK_GBS, 4), logit_copies=ncopy)
        del lcopies, xs_d, ws
        torch.cuda.empty_cache()
        print(f"# bench: sampler_r{R}_v{V}_k{k} measured", file=sys.stderr, flush=True)
    return res


if __name__ == "__main__":
    main()
