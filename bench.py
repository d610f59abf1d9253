#!/usr/bin/env python3
"""Throughput of the SVDQuant W4A4 linear layer on one MI355X.

One step is one whole layer call (svdq_linear: activation quantizer + block-
scaled FP4 GEMM with the fused low-rank epilogue) over one batch of seeded
synthetic input already resident in HBM.  The metric is effective TFLOP/s
counted as 2*M*N*K per call.  Prints one JSON line.

Default workload: the DiT MLP up-projection (M=4096, K=3072, N=12288, R=32),
the compute-bound headline shape.  Other workloads: --workload NAME.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_F16_MFMA_TFLOPS = 2500.0   # MI355X dense f16/bf16 matrix peak
PEAK_FP4_MFMA_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E peak
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dit_mlp_up")
    ap.add_argument("--sets", type=int, default=0, help="independent input sets cycled (0: enough to exceed 2x the MALL)")
    ap.add_argument("--graph", action="store_true", help="replay the timed steps from a captured HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-rows", type=int, default=256)
    ap.add_argument("--calib-copy", action="store_true", help="also run one 512 MiB device copy (counter calibration)")
    ap.add_argument("--mx", action="store_true",
                    help="the MXFP4 variant (E8M0 scale per 32, group-32 rotation) on the scaled FP4 matrix cores")
    ap.add_argument("--fwht", action="store_true",
                    help="the standalone block Hadamard transform, in place, on the workload's activation (M x K bf16)")
    ap.add_argument("--block", type=int, default=0, help="--fwht block size (default: the workload's, else 128)")
    return ap.parse_args()


def sha_of(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "gemm": ["w4a4_bit_quantized_amd/csrc/gemm.hip", "w4a4_bit_quantized_amd/csrc/gemm_common.h",
             "w4a4_bit_quantized_amd/csrc/device_common.h"],
    "gemm_skinny": ["w4a4_bit_quantized_amd/csrc/gemm_skinny.hip", "w4a4_bit_quantized_amd/csrc/device_common.h"],
    "gemm_mx": ["w4a4_bit_quantized_amd/csrc/gemm_mx.hip", "w4a4_bit_quantized_amd/csrc/gemm_common.h",
                "w4a4_bit_quantized_amd/csrc/device_common.h"],
    "gemm_skinny_mx": ["w4a4_bit_quantized_amd/csrc/gemm_skinny.hip", "w4a4_bit_quantized_amd/csrc/gemm_mx.hip",
                       "w4a4_bit_quantized_amd/csrc/device_common.h"],
    "hadamard": ["w4a4_bit_quantized_amd/csrc/hadamard.hip", "w4a4_bit_quantized_amd/csrc/device_common.h"],
    "quantize": ["w4a4_bit_quantized_amd/csrc/quantize.hip", "w4a4_bit_quantized_amd/csrc/device_common.h"],
}


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None if stale/missing.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by the factor the same counter
    gives for a device copy of known size."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(f"{kernel}:{workload}")
    cal = data.get("calibration")
    if not ent or not cal or ent.get("source_sha") != sha_of(KERNEL_SOURCES[kernel]):
        return None
    return 1024.0 * (ent["fetch_kib"] * cal["fetch_factor"] + ent["write_kib"] * cal["write_factor"])


def cpu_baseline(spec_name, cpu_rows, seconds, mx=False):
    """The oracle (CPU, NumPy) on a bounded row sample of the same workload."""
    import numpy as np
    from oracle import linear as olinear
    from oracle import mx as omx
    from oracle import quant as oquant
    from w4a4_bit_quantized_amd import synth
    lay = synth.make_layer(spec_name, seed=0)
    f = synth.as_f32(lay)
    B = 32 if mx else lay["B"]
    qweight_fn = omx.quantize_weight_mx if mx else oquant.quantize_weight
    linear_fn = omx.svdq_linear_mx if mx else olinear.svdq_linear
    qw, ws = qweight_fn(f["w"], f["smooth_factor"], B)  # offline, untimed
    rows = min(cpu_rows, lay["M"])
    layer = dict(qweight=qw, wscales=ws, **{k: f[k] for k in ("proj_down", "proj_up", "smooth_factor", "wcscales",
                                                              "wtscale")})
    x = np.ascontiguousarray(f["x"][:rows])
    reps, t_total = 0, 0.0
    while reps == 0 or t_total < seconds:
        t0 = time.perf_counter()
        linear_fn(x, layer, B)
        t_total += time.perf_counter() - t0
        reps += 1
    t = t_total / reps
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()
    flops = 2.0 * rows * lay["N"] * lay["K"]
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{rows} of {lay['M']} rows of {spec_name} (K={lay['K']}, N={lay['N']}, R={lay['R']}), "
                      f"whole layer (smooth, rotate, quantize, dequantize, float64 GEMM, epilogue), "
                      f"mean of {reps} runs, {t:.3f} s each; weight quantization untimed"}


def sleep_cycles(torch, stream, seconds):
    """Argument for torch.cuda._sleep that spins the GPU for about `seconds` (its clock, measured)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    torch.cuda._sleep(1 << 20)
    e1.record(stream)
    torch.cuda.synchronize()
    per_cycle = max(e0.elapsed_time(e1) * 1e-3, 1e-6) / (1 << 20)
    return int(min(seconds / per_cycle, 1 << 31))


def smi_state(flags):
    """rocm-smi's fields for the given query flags (power, performance level, clocks), or None."""
    import shutil
    import subprocess
    try:
        # rocm-smi is a Python script: run it with this interpreter rather than through its
        # "#!/usr/bin/env" line, so that no process replaces itself (under a profiler every child
        # process has initialised the GPU before its first instruction)
        tool = os.path.realpath(shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi")
        cmd = [sys.executable, tool] if tool.endswith(".py") else [tool]
        out = subprocess.run(cmd + flags + ["--json"], capture_output=True, text=True, timeout=20).stdout
        card = next(iter(json.loads(out).values()))
        return {k: v for k, v in card.items() if any(w in k.lower() for w in ("power", "perf", "sclk", "mclk", "fclk"))}
    except Exception:  # pragma: no cover - tool missing or unparsable output
        return None


def run_environment(torch):
    """ROCm version, GPU, and the power state rocm-smi reports (None where unavailable)."""
    props = torch.cuda.get_device_properties(0)
    env = {"rocm": None, "gpu": getattr(props, "gcnArchName", props.name), "cus": props.multi_processor_count,
           "torch": torch.__version__, "power": None}
    try:
        with open(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), ".info", "version")) as f:
            env["rocm"] = f.read().strip()
    except OSError:
        pass
    env["power"] = smi_state(["--showpower", "--showperflevel", "--showmaxpower", "--showclocks"])
    return env


def cpu_baseline_fwht(M, K, block, seconds):
    """The oracle's standalone transform (CPU, NumPy) on a bounded row sample of the same tensor shape."""
    import numpy as np
    from oracle import hadamard as oh
    rng = np.random.default_rng(0)
    rows = 64
    x = oh.from_f32(rng.standard_normal((rows, K)).astype(np.float32), "bf16")
    t0 = time.perf_counter()
    reps = 0
    while True:
        oh.hadamard_transform(x, block, "bf16")
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    t = (time.perf_counter() - t0) / reps
    return {"value": round(2 * rows * K * 2 / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of {M} rows of {M} x {K} bf16, blocks of {block}, mean of {reps} runs, {t:.3f} s each "
                      f"(NumPy, one thread)"}


def main_fwht(args):
    """The standalone block Hadamard transform, in place, over input sets exceeding twice the MALL."""
    import ctypes
    import torch

    import w4a4_bit_quantized_amd as w4
    from w4a4_bit_quantized_amd import binding, synth

    if not os.path.exists(binding.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    lib = w4.load_library()
    spec = synth.WORKLOADS[args.workload]
    M, K = spec["M"], spec["K"]
    block = args.block or spec["B"] or 128
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    per_set = M * K * 2
    nsets = args.sets or max(1, -(-2 * MALL_BYTES // per_set))
    g = torch.Generator(device=dev).manual_seed(0)
    sets = [torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16) for _ in range(nsets)]
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    fargs = [(ctypes.c_void_p(t.data_ptr()), K, ctypes.c_void_p(t.data_ptr()), K, M, K, block, binding.DTYPE_BF16, sp)
             for t in sets]

    def step(i):
        st = lib.w4a4_hadamard_transform(*fargs[i % nsets])
        if st:
            raise RuntimeError(f"w4a4_hadamard_transform failed with status {st}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(sleep_cycles(torch, stream, 2e-3 + 20e-6 * args.steps))
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    k_us = 1e3 * ev0.elapsed_time(ev1) / args.steps
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    if args.calib_copy:
        a = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
    nbytes = 2 * M * K * 2  # every element read and written once
    ach = nbytes / (k_us * 1e-6) / 1e9
    tr = traffic_from_profile("hadamard", args.workload)
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "kernel": "hadamard", "traffic": None if tr is None else round(tr)}
    cpu = None if args.no_cpu_baseline else cpu_baseline_fwht(M, K, block, args.cpu_seconds)
    line = {
        "metric": "block Hadamard transform GB/s (bf16 read + write) and % of HBM roofline",
        "value": round(nbytes / (wall_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall_ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "storage": "bf16", "data": "synthetic",
        "config": {"workload": args.workload + "_fwht", "M": M, "K": K, "block": block, "input_sets": nsets},
        "kernels": {"hadamard": {"avg_us": round(k_us, 3), "algorithmic_bytes": nbytes, "achieved_GBps": round(ach, 1)}},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the layer's sharding across GPUs "
              f"is a design, not built here)", file=sys.stderr)
        sys.exit(2)
    if args.fwht:
        return main_fwht(args)

    import ctypes
    import numpy as np
    import torch

    import w4a4_bit_quantized_amd as w4
    from w4a4_bit_quantized_amd import binding, synth

    if not os.path.exists(binding.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    lib = w4.load_library()
    spec = synth.WORKLOADS[args.workload]
    M, K, N, R, B = spec["M"], spec["K"], spec["N"], spec["R"], spec["B"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.mx:
        B = 32  # the MX variant rotates in blocks of 32 (its weights are quantized with the same rotation)
    ws_bytes = w4.svdq_linear_mx_workspace_bytes if args.mx else w4.svdq_linear_workspace_bytes
    sgroup = 32 if args.mx else 16
    per_set = M * K * 2 + N * K // 2 + N * K // sgroup + M * N * 2 + ws_bytes(M, K, R)
    nsets = args.sets or max(1, -(-2 * MALL_BYTES // per_set))

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    sets = []
    for s in range(nsets):
        lay = synth.make_layer(args.workload, seed=s)
        wdev = bf(lay["w"])
        lam = bf(lay["smooth_factor"])
        quantize_weight = w4.svdq_quantize_weight_mx if args.mx else w4.svdq_quantize_weight
        qw, ws = quantize_weight(wdev, lam, B)  # offline weight quantization on the GPU
        del wdev
        t = dict(x=bf(lay["x"]), qweight=qw, wscales=ws, proj_down=bf(lay["proj_down"]), proj_up=bf(lay["proj_up"]),
                 smooth_factor=lam, wcscales=bf(lay["wcscales"]), wtscale=bf(lay["wtscale"]))
        t["y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        nbytes = ws_bytes(M, K, R)
        t["ws"] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        # workspace views used by the two-entry-point breakdown loop (same layout as svdq_linear's)
        a256 = lambda v: (v + 255) // 256 * 256
        srows = (M + 3) // 4 * 4 if args.mx else M
        t["qact"] = t["ws"][: M * K // 2]
        t["ascales"] = t["ws"][a256(M * K // 2): a256(M * K // 2) + K // sgroup * srows]
        off = a256(M * K // 2) + a256(K // sgroup * srows)
        t["lora"] = t["ws"][off: off + M * R * 4].view(torch.float32)
        sets.append(t)
        del lay
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda tt: ctypes.c_void_p(tt.data_ptr())
    lin_args = [(P(t["x"]), P(t["qweight"]), P(t["wscales"]), P(t["proj_down"]), P(t["proj_up"]),
                 P(t["smooth_factor"]), P(t["wcscales"]), P(t["wtscale"]), M, N, K, R, B, P(t["y"]), P(t["ws"]),
                 t["ws"].numel(), sp) for t in sets]
    q_args = [(P(t["x"]), P(t["smooth_factor"]), P(t["proj_down"]), M, K, R, B, P(t["qact"]), P(t["ascales"]),
               P(t["lora"]), sp) for t in sets]
    g_args = [(P(t["qact"]), P(t["ascales"]), P(t["lora"]), P(t["qweight"]), P(t["wscales"]), P(t["proj_up"]),
               P(t["wcscales"]), P(t["wtscale"]), M, N, K, R, P(t["y"]), sp) for t in sets]

    f_linear = lib.svdq_linear_mx if args.mx else lib.svdq_linear
    f_quant = lib.svdq_quantize_act_mx if args.mx else lib.svdq_quantize_act
    f_gemm = lib.svdq_gemm_lowrank_mx if args.mx else lib.svdq_gemm_lowrank

    def step(i):
        st = f_linear(*lin_args[i % nsets])
        if st:
            raise RuntimeError(f"svdq_linear failed with status {st}")

    env = run_environment(torch)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        gs = torch.cuda.Stream(dev)
        gs.wait_stream(stream)
        with torch.cuda.stream(gs):
            gsp = ctypes.c_void_p(gs.cuda_stream)
            with torch.cuda.graph(graph, stream=gs):
                for i in range(args.steps):
                    a = list(lin_args[i % nsets])
                    a[-1] = gsp
                    f_linear(*a)
        stream.wait_stream(gs)
        torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    gpu_ms = ev0.elapsed_time(ev1) / args.steps

    # rocm-smi's power and clock state right after the timed steps
    smi_after = smi_state(["--showpower", "--showclocks"])

    # Per-kernel durations: the same two kernels through the two-entry-point form, each launched
    # back to back (one HIP event pair around the whole run of launches: a pair around every
    # launch would add the dispatch gap to kernels of a few microseconds), 5 runs of at least 100
    # launches, median.  Every launch of a run works on buffers that no other launch of the run
    # touches, so each kernel reads its inputs from HBM (cold), as it does inside the layer: the
    # quantizer runs cycle through copies of x (same values, distinct buffers), the GEMM runs
    # through the input sets (their working set exceeds twice the 256 MB Infinity Cache).
    calls = max(args.steps, 100)
    qparts = 1 if M > 32 or K < 1024 else min(K // 512, 8)  # the layer's K split of the quantizer
    q_in = max(1, min(calls, -(-2 * MALL_BYTES // (M * K * 2 + M * K // 2 + M * K // sgroup))))
    srows = (M + 3) // 4 * 4 if args.mx else M
    x_copies = [sets[i % nsets]["x"].clone() for i in range(q_in)]
    q_out = [(torch.empty(M * K // 2, dtype=torch.uint8, device=dev),
              torch.empty(K // sgroup * srows, dtype=torch.uint8, device=dev),
              torch.empty(M * max(R, 1), dtype=torch.float32, device=dev)) for _ in range(q_in)]
    qc_args = [(P(x_copies[i]), P(sets[i % nsets]["smooth_factor"]), P(sets[i % nsets]["proj_down"]), M, K, R, B,
                P(q_out[i][0]), P(q_out[i][1]), P(q_out[i][2]), sp) for i in range(q_in)]
    torch.cuda.synchronize()

    def timed_run(fn, argl, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # a bounded spin kernel first, so that the host queues the whole run before the GPU reaches it
        torch.cuda._sleep(sleep_cycles(torch, stream, 2e-3 + 40e-6 * n))
        e0.record(stream)
        for i in range(n):
            fn(*argl[i % len(argl)])
        e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n

    q_runs, g_runs = [], []
    for _ in range(5):  # alternating: each GEMM run streams far more than the cache holds
        q_runs.append(timed_run(f_quant, qc_args, calls))
        g_runs.append(timed_run(f_gemm, g_args, calls))
    q_us, g_us = float(np.median(q_runs)), float(np.median(g_runs))

    if args.calib_copy:
        a = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    flops = 2.0 * M * N * K
    value = flops / (wall_ms * 1e-3) / 1e12
    q_bytes = M * K * 2 + K * 2 + K * R * 2 + M * K // 2 + M * K // sgroup + M * R * 4
    g_bytes = M * K // 2 + M * K // sgroup + M * R * 4 + N * K // 2 + N * K // sgroup + N * R * 2 + N * 2 + M * N * 2
    kernels = {
        "quantize_act": {"avg_us": round(q_us, 3), "runs_us": [round(v, 3) for v in q_runs], "calls_per_run": calls,
                         "cache": "cold", "algorithmic_bytes": q_bytes, "entry": "svdq_quantize_act" + (
                             " (one K part: inside svdq_linear the quantizer splits K into %d parts)" % qparts
                             if qparts > 1 else ""),
                         "achieved_GBps": round(q_bytes / (q_us * 1e-6) / 1e9, 1)},
        "gemm_lowrank": {"avg_us": round(g_us, 3), "runs_us": [round(v, 3) for v in g_runs], "calls_per_run": calls,
                         "cache": "cold", "algorithmic_bytes": g_bytes, "flops": flops,
                         "achieved_TFLOPs": round(flops / (g_us * 1e-6) / 1e12, 1),
                         "achieved_GBps": round(g_bytes / (g_us * 1e-6) / 1e9, 1)},
    }
    compute_bound = M >= 256
    if compute_bound and args.mx:  # the scaled FP4 instruction: priced against the FP4 peak
        ach = flops / (g_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_FP4_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_FP4_MFMA_TFLOPS, 4), "kernel": "gemm_lowrank"}
    elif compute_bound:
        ach = flops / (g_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_F16_MFMA_TFLOPS, 4), "kernel": "gemm_lowrank",
                "frac_of_fp4_peak": round(ach / PEAK_FP4_MFMA_TFLOPS, 4)}
    else:
        ach = g_bytes / (g_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "kernel": "gemm_lowrank"}
    if args.mx:
        gemm_kernel = "gemm_skinny_mx" if M <= 16 and K % 512 == 0 and K <= 5120 and R <= 64 else "gemm_mx"
    else:
        gemm_kernel = "gemm_skinny" if M <= 32 else "gemm"
    roof["kernel"] = gemm_kernel
    tr = traffic_from_profile(gemm_kernel, args.workload)
    roof["traffic"] = None if tr is None else round(tr)

    # whole-layer figure for the weight-streaming regime: the minimum bytes of one fused pass
    # (x, weights and scales, low-rank factors, smooth_factor, wcscales, y) over the step time
    layer_bytes = (M * K * 2 + N * K // 2 + N * K // sgroup + (K + N) * R * 2 + K * 2 + N * 2 + M * N * 2)
    layer = {"min_bytes": layer_bytes, "us_per_step": round(wall_ms * 1e3, 3),
             "achieved_GBps": round(layer_bytes / (wall_ms * 1e-3) / 1e9, 1),
             "hbm_frac": round(layer_bytes / (wall_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, args.cpu_rows, args.cpu_seconds, args.mx)

    line = {
        "metric": "W4A4 linear effective TFLOP/s (2MNK) and % of FP4-MFMA/HBM roofline",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5), "gpu_ms_per_step": round(gpu_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp4" if args.mx else "f16",
        "storage": "fp4 e2m1 + e8m0 per 32 (mxfp4)" if args.mx else "fp4 e2m1 + e4m3 per 16 (nvfp4)",
        "data": "synthetic",
        "config": {"workload": args.workload + ("_mx" if args.mx else ""), "M": M, "K": K, "N": N, "R": R,
                   "hadamard_block": B, "input_sets": nsets, "graph": bool(args.graph)},
        "frac_of_fp4_peak": round(value / PEAK_FP4_MFMA_TFLOPS, 4),
        "layer": layer, "kernels": kernels, "roofline": roof, "cpu_baseline": cpu,
        "env": dict(env, power_after_timed=smi_after),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
