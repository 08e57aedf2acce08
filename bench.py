"""Benchmark: fused exact attention on one MI355X.

One step = one forward call over the whole workload (every head, every
query block, the full key loop), inputs resident in device memory.  The
default workload is the long-sequence causal case B=1, H=16, N=16384,
d=128, bf16.  Throughput counts 4*B*H*N^2*d FLOPs, halved for causal.
``--pass bwd`` times one backward call (attn_bwd: dQ, dK, dV from the
forward's O and LSE and a seeded dO) instead, counted as 2.5 times the
forward's FLOPs.

Steps shorter than 0.2 ms (image-model rows, one-token decode) are launch
bound: after the direct timing, the same steps are captured once into a HIP
graph and the graph is replayed; ``config.launch`` says which was reported
(``--launch direct`` keeps one launch per step).

Prints one JSON line per workload.  ``roofline`` compares the kernel's rate
(HIP events around the timed launches, on the launch stream) with the
published dense matrix-core peak; ``traffic`` comes from a committed counter
summary only while the kernel sources it was measured on are unchanged (else
null).  ``cpu_baseline`` times the float64 CPU oracle on a bounded sample of
the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK = {"bf16": 2500.0, "fp8": 5000.0,          # published MI355X dense matrix-core TFLOP/s
        "f32": 157.3}                            # published MI355X float32 vector TFLOP/s
HBM_PEAK_GBS = 8000.0                            # published MI355X HBM3E bandwidth
INPUT_SET_BYTES = 512 * 10 ** 6                  # > 2x the 256 MB last-level cache
KERNEL_SOURCES = {
    "f32": ["exact_attention_127_amd/csrc/attn_simple.hip",
            "exact_attention_127_amd/csrc/common.h"],
    "bf16": ["exact_attention_127_amd/csrc/attn_mfma_bf16.hip",
             "exact_attention_127_amd/csrc/device_util.h",
             "exact_attention_127_amd/csrc/common.h"],
    "fp8": ["exact_attention_127_amd/csrc/attn_fp8.hip",
            "exact_attention_127_amd/csrc/device_util.h",
            "exact_attention_127_amd/csrc/common.h"],
    "mxfp8": ["exact_attention_127_amd/csrc/attn_fp8.hip",
              "exact_attention_127_amd/csrc/device_util.h",
              "exact_attention_127_amd/csrc/common.h"],
    "w4a16": ["exact_attention_127_amd/csrc/w4a16.hip",
              "exact_attention_127_amd/csrc/common.h"],
    "bwd": ["exact_attention_127_amd/csrc/attn_bwd.hip",
            "exact_attention_127_amd/csrc/device_util.h",
            "exact_attention_127_amd/csrc/common.h"],
}
# the backward's products: dV, dP, dQ, dK and the recomputed S, each the size of
# one forward product, i.e. 2.5 times the forward's algorithmic FLOPs
BWD_FLOP_FACTOR = 2.5


def kernel_hash(kind: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str, kind: str):
    """Per-launch HBM bytes from a committed counter summary, if still valid."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_hash") != kernel_hash(kind):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(inp, budget_s: float = 12.0) -> dict:
    """The float64 oracle on whole heads of the workload until ~budget_s elapse."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    w = inp["workload"]
    rows = np.arange(w.N)
    flops_head = w.flops / (w.B * w.H)
    # whole heads in order, starting over when a small workload is done
    # before the budget
    t0 = time.perf_counter()
    done = 0
    while True:
        b, h = divmod(done % (w.B * w.H), w.H)
        oracle.attention_rows(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                              inp["scale"], w.causal, rows)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done * flops_head / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} head evaluations over the workload's {w.B * w.H} heads (all {w.N} "
                      f"query rows each), float64 numpy, {dt:.1f} s"}


def cpu_baseline_bwd(inp, do, budget_s: float = 12.0) -> dict:
    """The float64 gradient oracle on whole heads until ~budget_s elapse."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    w = inp["workload"]
    flops_head = algorithmic_flops(w, "bwd") / (w.B * w.H)
    t0 = time.perf_counter()
    done = 0
    while True:
        b, h = divmod(done % (w.B * w.H), w.H)
        oracle.attention_backward_head(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                                       do[b, h], inp["scale"], w.causal)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done * flops_head / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} head evaluations over the workload's {w.B * w.H} heads (dQ, dK, dV "
                      f"of all {w.N} rows each), float64 numpy, {dt:.1f} s"}


def timed(step, stream, steps, warmup):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t_w = time.perf_counter()            # let the clocks settle: about a second of work
    while time.perf_counter() - t_w < 1.0:
        step()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, ev0.elapsed_time(ev1) / steps


# Steps shorter than this are launch bound: the host's per-launch cost and the
# gaps between launches are then a visible share of the step, so the timed
# steps are captured once into a HIP graph and replayed (each step is still
# executed; tests/test_graph_gpu.py checks replays against eager launches).
GRAPH_BELOW_MS = 0.2


def timed_graph(make_step, steps, warmup):
    """As timed(), with the K timed steps captured into one HIP graph on a
    side stream (default priority) and replayed once."""
    import torch
    side = torch.cuda.Stream()
    gstep = make_step(side)
    for _ in range(warmup):
        gstep()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(steps):
            gstep()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        t_w = time.perf_counter()            # let the clocks settle: about a second of work
        while time.perf_counter() - t_w < 1.0:
            g.replay()
            torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(side)
        g.replay()
        ev1.record(side)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    return wall * 1e3 / steps, ev0.elapsed_time(ev1) / steps


def timed_steps(step, make_step, stream, args):
    """Direct launches; then, for a launch-bound step that can be rebuilt on
    another stream (make_step), the same steps replayed from a HIP graph.
    Returns (ms_per_step, kernel_ms, launch)."""
    ms, kms = timed(step, stream, args.steps, args.warmup)
    if make_step is None or args.launch == "direct" or (args.launch == "auto" and ms >= GRAPH_BELOW_MS):
        return ms, kms, "direct"
    try:
        gms, gkms = timed_graph(make_step, args.steps, args.warmup)
    except RuntimeError as e:
        print(f"bench: graph capture failed ({e}); reporting direct launches", file=sys.stderr)
        return ms, kms, "direct"
    return gms, gkms, "hip_graph"


def algorithmic_bytes(w, kind: str) -> int:
    """Forward: Q, K, V read once (2 B per element in bf16, 1 B in fp8), O
    (bf16) and LSE (float32) written once; MXFP8 also reads one scale byte per
    32 channels of every Q, K and V row.  Backward: Q, K, V, O, dO and LSE
    read once, dQ, dK, dV written once, the row statistic D written and read."""
    if kind == "bwd":
        return w.B * w.H * w.N * (5 * 2 * w.d + 4 + 3 * 2 * w.d + 8)
    if kind == "f32":
        return w.B * w.H * w.N * (4 * 4 * w.d + 4)
    in_bytes = 2 if kind == "bf16" else 1
    scale_bytes = 3 * (w.d // 32) if kind == "mxfp8" else 0
    return w.B * w.H * w.N * (3 * in_bytes * w.d + scale_bytes + 2 * w.d + 4)


def algorithmic_flops(w, kind: str) -> float:
    return w.flops * (BWD_FLOP_FACTOR if kind == "bwd" else 1.0)


def roofline(w, kind: str, kernel_ms: float, peak_tflops: float):
    """The bound that applies to one launch of workload ``w``: HBM when moving
    its algorithmic bytes at peak bandwidth takes longer than its FLOPs at
    peak compute rate, else the compute units (matrix cores; the float32
    vector ALUs for the float32 path)."""
    alg_bytes = algorithmic_bytes(w, kind)
    flops = algorithmic_flops(w, kind)
    if alg_bytes / (HBM_PEAK_GBS * 1e9) > flops / (peak_tflops * 1e12):
        roof = {"bound": "hbm", "achieved": round(alg_bytes / (kernel_ms * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "alu" if kind == "f32" else "mfma",
                "achieved": round(flops / (kernel_ms * 1e-3) / 1e12, 2),
                "peak": round(peak_tflops, 1), "unit": "TFLOP/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    return roof, alg_bytes


def run_workload(name, args, fp8_scales="tile"):
    import torch
    import exact_attention_127_amd as A
    from seeded_inputs import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    stream = torch.cuda.current_stream()
    extra = {}
    extra_cfg = {}
    make_step = None      # set where a step can be rebuilt on another stream (graph capture)
    if args.pass_ == "bwd":
        if w.dtype != "bf16":
            raise SystemExit(f"the backward pass takes bf16 workloads, not {name}")
        from seeded_inputs import make_output_grad
        kind = "bwd"
        q, k, v = (torch.from_numpy(inp[x]).to(dev).to(torch.bfloat16).contiguous() for x in "qkv")
        do_np = make_output_grad(w)
        dout = torch.from_numpy(do_np).to(dev).to(torch.bfloat16).contiguous()
        o, lse = A.attn_fwd(q, k, v, scale=w.scale, causal=w.causal, stream=stream)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        delta = torch.empty_like(lse)

        def step():
            A.attn_bwd(q, k, v, o, dout, lse, dq=dq, dk=dk, dv=dv, delta=delta, scale=w.scale,
                       causal=w.causal, stream=stream)
        peak = PEAK["bf16"]
    elif w.dtype in ("bf16", "f32"):
        kind = w.dtype
        peak = PEAK[kind]
        tdt = torch.bfloat16 if kind == "bf16" else torch.float32
        q, k, v = (torch.from_numpy(inp[x]).to(dev).to(tdt).contiguous() for x in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        # an HBM-bound launch cycles through copies of its buffers, more than
        # 512 MB in all, so the 256 MB last-level cache cannot serve them
        bufs = [(q, k, v, o, lse)]
        if roofline(w, kind, 1.0, peak)[0]["bound"] == "hbm":
            n_sets = -(-INPUT_SET_BYTES // algorithmic_bytes(w, kind))
            bufs += [tuple(t.clone() for t in bufs[0]) for _ in range(n_sets - 1)]
        extra_cfg["input_sets"] = len(bufs)
        # arguments checked once per buffer set: a launch is then one C call,
        # so the host keeps up with the 20-30 us kernels of short sequences
        def make_step(st):
            launchers = [A.attn_fwd_launcher(qi, ki, vi, oi, li, scale=w.scale, causal=w.causal,
                                             stream=st) for (qi, ki, vi, oi, li) in bufs]
            turn = [0]

            def one():
                launchers[turn[0] % len(launchers)]()
                turn[0] += 1
            return one
        step = make_step(stream)
    elif w.dtype == "fp8":
        mx = fp8_scales == "mx"
        kind = "mxfp8" if mx else "fp8"
        prepare = A.attn_mxfp8_prepare if mx else A.attn_fp8_prepare
        forward = A.attn_fwd_mxfp8 if mx else A.attn_fwd_fp8
        qf, kf, vf = (torch.from_numpy(inp[x]).to(dev).contiguous() for x in "qkv")
        R = torch.from_numpy(inp["R"]).to(dev).contiguous()
        q8, k8, v8, sq, sk, sv = prepare(qf, kf, vf, R)
        o = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        _, prep_ms = timed(lambda: prepare(qf, kf, vf, R), stream, 3, 1)
        prep_bytes = (3 * qf.numel() * 4 + 3 * qf.numel() + 3 * sq.numel() * sq.element_size()
                      + R.numel() * 4)
        extra["prepare"] = {"ms": round(prep_ms, 4), "GB_per_s": round(prep_bytes / prep_ms / 1e6, 1)}

        def step():
            forward(q8, k8, v8, sq, sk, sv, o=o, lse=lse, scale=w.scale, causal=w.causal,
                    stream=stream)
        # the dense fp8 peak; P V runs on fp16 (per-tile scales) or bf16
        # (MXFP8) matrix cores, so a time-weighted peak of the two halves
        # is reported beside it
        peak = PEAK["fp8"]
        extra_cfg["blended_peak_tflops"] = round(1.0 / (0.5 / PEAK["fp8"] + 0.5 / PEAK["bf16"]), 1)
    else:
        raise SystemExit(f"bench.py times the bf16 and fp8 workloads, not {name}")

    ms_per_step, kernel_ms, launch = timed_steps(step, make_step, stream, args)
    extra_cfg["launch"] = launch
    flops = algorithmic_flops(w, kind)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    roof, alg_bytes = roofline(w, kind, kernel_ms, peak)
    if "blended_peak_tflops" in extra_cfg and roof["bound"] == "mfma":
        roof["frac_of_blended_peak"] = round(roof["achieved"] / extra_cfg["blended_peak_tflops"], 4)
    if kind == "f32":
        extra_cfg["latency_us"] = round(kernel_ms * 1e3, 2)
    line = {
        "metric": ("attn fwd TFLOP/s + % of bf16 MFMA peak, B=1 H=16 N=16384 d=128 causal"
                   if name == "long_causal_16k" and kind != "bwd" else
                   f"attn {'bwd' if kind == 'bwd' else 'fwd'} TFLOP/s, {name}"
                   + (", MXFP8 scales" if kind == "mxfp8" else "")),
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "seed": w.seed, "flops_per_step": flops,
                   "pass": "bwd" if kind == "bwd" else "fwd",
                   **({"fp8_scales": fp8_scales} if w.dtype == "fp8" else {}),
                   "pct_of_peak": round(100 * tflops / peak, 2), **extra_cfg},
        "roofline": {**roof, "traffic": traffic_from_profile(w.name + {"bwd": "_bwd", "mxfp8": "_mx"}.get(kind, ""), kind),
                     "algorithmic_bytes": alg_bytes,
                     "kernel_ms": round(kernel_ms, 4), "kernel_hash": kernel_hash(kind)},
    }
    line.update(extra)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_bwd(inp, do_np) if kind == "bwd" else cpu_baseline(inp)
    print(json.dumps(line), flush=True)


def cpu_baseline_w4(inp, budget_s: float = 12.0) -> dict:
    """The float64 W4A16 oracle on blocks of output columns until ~budget_s elapse."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    w = inp["workload"]
    cols_per = 512
    # blocks of output columns in order, starting over at the end
    t0 = time.perf_counter()
    done = 0
    while True:
        c0 = done % w.N
        cols = np.arange(c0, min(w.N, c0 + cols_per))
        oracle.w4a16_rows(inp["x"], inp["qweight"], inp["scales"], inp["zeros"], w.G, cols)
        done += len(cols)
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    bytes_done = w.bytes * done / w.N
    return {"value": bytes_done / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} output-column evaluations over the workload's {w.N} columns (all "
                      f"{w.M} tokens each), float64 numpy, {dt:.1f} s"}


def run_w4(name, args):
    """One launch of w4a16_gemm per step; HBM-bound, so the buffers cycle
    through copies totalling more than 512 MB."""
    import numpy as np
    import torch
    import exact_attention_127_amd as A
    from seeded_inputs import W4_WORKLOADS, make_w4a16_inputs

    w = W4_WORKLOADS[name]
    dev = torch.device("cuda:0")
    inp = make_w4a16_inputs(w)
    stream = torch.cuda.current_stream()
    base = (torch.from_numpy(inp["x"]).to(dev),
            torch.from_numpy(inp["qweight"].view(np.int32)).to(dev),
            torch.from_numpy(inp["scales"]).to(dev),
            torch.from_numpy(inp["zeros"]).to(dev),
            torch.empty((w.M, w.N), dtype=torch.float16, device=dev))
    n_sets = -(-INPUT_SET_BYTES // w.bytes)
    bufs = [base] + [tuple(t.clone() for t in base) for _ in range(n_sets - 1)]
    # arguments checked once per buffer set; a launch is then one C call
    def make_step(st):
        launchers = [A.w4a16_gemm_launcher(x, q, sc, z, y, group=w.G, stream=st) for (x, q, sc, z, y) in bufs]
        turn = [0]

        def one():
            launchers[turn[0] % len(launchers)]()
            turn[0] += 1
        return one

    ms_per_step, kernel_ms, launch = timed_steps(make_step(stream), make_step, stream, args)
    gbs = w.bytes / (ms_per_step * 1e-3) / 1e9
    achieved = w.bytes / (kernel_ms * 1e-3) / 1e9
    line = {
        "metric": f"w4a16 decode product GB/s (algorithmic bytes), {name}",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int4 weights, fp16 activations",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "group": w.G, "seed": w.seed,
                   "bytes_per_step": w.bytes, "flops_per_step": w.flops, "input_sets": len(bufs),
                   "launch": launch,
                   "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(w.name, "w4a16"),
                     "algorithmic_bytes": w.bytes, "kernel_ms": round(kernel_ms, 4),
                     "kernel_hash": kernel_hash("w4a16")},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_w4(inp)
    print(json.dumps(line), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_causal_16k",
                    help="workload name, or 'all' for one line per bf16/fp8 workload")
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward pass (default) or the backward pass (bf16 workloads)")
    ap.add_argument("--fp8-scales", choices=("tile", "mx"), default="tile",
                    help="fp8 workloads: one float32 scale per 128-token tile (default) or one "
                         "power-of-two scale per 32 channels of a token (MXFP8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--launch", choices=("auto", "direct", "graph"), default="auto",
                    help="auto: steps shorter than %.1f ms are replayed from a HIP graph "
                         "(forward and W4A16); direct: one launch per step; graph: always replay"
                         % GRAPH_BELOW_MS)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of 1 GiB per step (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(heads are independent, so several GPUs would each run this kernel on "
              "their share of heads)", file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 2, "copy_bytes_written": dst.numel() * 2,
                          "launches": args.warmup + args.steps}))
        return 0
    if args.workload != "all":
        runs = [(args.workload, args.fp8_scales)]
    else:
        runs = [(n, "tile") for n in ("long_causal_16k", "vit_b16_batch64", "llm_layer_4k")]
        if args.pass_ == "fwd":
            runs.insert(1, ("vit_b16_single", "tile"))
        if args.pass_ == "fwd":
            runs += [("fp8_outliers_8k", "tile"), ("fp8_outliers_8k", "mx"),
                     ("w4a16_decode_70b", None), ("w4a16_batch16_70b", None)]
    for n, fmt in runs:
        if n.startswith("w4a16"):
            if args.pass_ == "bwd":
                raise SystemExit("the W4A16 product has no backward pass here")
            run_w4(n, args)
        else:
            run_workload(n, args, fmt)
    return 0


if __name__ == "__main__":
    sys.exit(main())
