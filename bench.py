#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = the whole path over one batch of resident synthetic inputs:
fa_fwd (forward kernel) followed by the backward kernels (dQ, which forms
rowsum(dO.O) itself on this path, then dK/dV), each launched through the C ABI
on torch's current stream.

Default workload: long-context causal fp16 attention, B=1, H=16,
S=16384, D=128, Q/K/V/dO iid N(0,1) rounded to fp16.

FLOP accounting: forward = 4*B*H*Sq*Sk*D, halved when causal ("FlashAttention-2
from PyTorch to Triton", the benchmark harness's attn_flops); forward+backward
= 3.5x forward (backward counted as 2.5x forward).  The roofline object
reports the dominant kernel against the dense fp16 MFMA peak of MI355X.

Beside the headline figure the line carries: the same step in bfloat16, the
peak memory beyond the inputs of one autograd forward + backward, the measured
dense fp16 MFMA and v_exp_f32 rates of the device (library probes), the length
sweep (S = 512 ... 16384 with B = 16384/S, causal and not, forward and
forward+backward TFLOP/s and fraction of peak), the CPU oracle timed on a
bounded sample of the workload, and the pages' own T4 figures as context.

Prints ONE JSON line.  ``--gpus`` above 1 is refused: this build runs on one
GPU only (attention heads shard across GPUs with no communication).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

MFMA_PEAK_F16 = 2516.6  # TFLOP/s, dense fp16, MI355X (256 CU x 4096 flop/clk x 2.4 GHz)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # About half a second of untimed steps: the GPU needs that long under this
    # load to reach its working clock (a first timed pass after idle reads up
    # to a quarter slow).
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=3,
                    help="heads of the workload the CPU oracle times (bounded sample)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy (for scaling HBM counters)")
    ap.add_argument("--no-length-sweep", action="store_true",
                    help="skip the fp16 length sweep (S = 512 ... 16384, causal and not)")
    ap.add_argument("--sweep", default="",
                    help="optional path: also write the length sweep's records there, one JSON line each")
    ap.add_argument("--no-bf16", action="store_true",
                    help="skip the secondary bfloat16 timing of the same workload")
    return ap.parse_args()


def fwd_flops(B, H, Sq, Sk, D, causal):
    f = 4.0 * B * H * Sq * Sk * D
    return f / 2 if causal else f


def make_device_inputs(case, torch):
    from exact_attention_88_amd import workloads as W
    x = W.make_inputs(case)
    dev = {n: torch.from_numpy(a.copy()).to("cuda") for n, a in x.items()}
    if case.dtype == "bf16":  # float32 arrays holding bfloat16 values: exact cast
        dev = {n: t.to(torch.bfloat16) for n, t in dev.items()}
    return x, dev


def time_path(fa, torch, case, dev, steps, warmup):
    """Time `steps` full passes; per-kernel durations from HIP events recorded
    on the stream the kernels run on (torch's current stream)."""
    B, H, Sq, Sk, D = case.B, case.H, case.Sq, case.Sk, case.D
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    sc = case.scale

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fa_fwd(q, k, v, case.causal, sc, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        # rowsum(dO.O) (nothing where the dQ kernel forms it), dQ, dK/dV: the
        # order fa_bwd runs them in.
        for j, stage in enumerate((0, 2, 1)):
            fa.fa_bwd_stage(stage, -1, q, k, v, o, do, lse, case.causal, sc, dq=dq, dk=dk, dv=dv,
                            delta=delta)
            if ev is not None:
                ev[2 + j].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ("fwd", "bwd_pre", "bwd_dq", "bwd_dkdv")
    per = {n: [] for n in names}
    for ev in evs:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]))
    avg = {n: sum(v) / len(v) for n, v in per.items()}
    return wall, avg


def length_sweep(fa, torch, steps, warmup):
    """Forward and forward+backward TFLOP/s and fraction of the dense fp16
    MFMA peak at S = 512 ... 16384 (fp16, H = 16, D = 128, B = 16384/S: 16k
    tokens per call), causal and not.  Causal and non-causal cases of one
    length share their seeded inputs."""
    from exact_attention_88_amd import workloads as W
    out, cached = [], {}
    for sc in W.sweep_cases():
        key = (sc.Sq, sc.seed)
        if key not in cached:
            cached.clear()
            cached[key] = make_device_inputs(sc, torch)[1]
        wall, avg = time_path(fa, torch, sc, cached[key], steps, warmup)
        ff = fwd_flops(sc.B, sc.H, sc.Sq, sc.Sk, sc.D, sc.causal)
        fwd_tf = ff / (avg["fwd"] * 1e-3) / 1e12
        fb_tf = 3.5 * ff / (wall / steps) / 1e12
        out.append({"S": sc.Sq, "B": sc.B, "causal": sc.causal,
                    "fwd_tflops": round(fwd_tf, 1), "fwd_frac_of_peak": round(fwd_tf / MFMA_PEAK_F16, 4),
                    "fwdbwd_tflops": round(fb_tf, 1),
                    "fwdbwd_frac_of_peak": round(fb_tf / MFMA_PEAK_F16, 4),
                    "ms_per_step": round(wall / steps * 1e3, 4),
                    "kernel_ms": {n: round(v, 4) for n, v in avg.items()}})
    cached.clear()
    return out


def probe_rates(fa, torch):
    """Measured ceilings on this device: dense fp16 MFMA TFLOP/s and v_exp_f32
    exponentials per second (the library's probes, timed with HIP events on
    the stream they run on after a warm-up launch)."""
    n = fa.fa_probe_threads()
    sink = torch.empty(n, device="cuda")
    out = {}
    for kind, iters in ((0, 4000), (1, 20000)):
        fa.fa_probe(kind, iters, sink)
        best = float("inf")
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fa.fa_probe(kind, iters, sink)
            e1.record()
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e-3)
        if kind == 0:
            tf = (n // 64) * iters * 4 * 32768 / best / 1e12
            out["mfma_f16_tflops"] = round(tf, 1)
            out["mfma_f16_frac_of_peak"] = round(tf / MFMA_PEAK_F16, 4)
        else:
            out["exp2_per_s"] = float(f"{n * iters * 8 / best:.4g}")
    return out


# The pages' own figures for this method (NVIDIA T4, Triton; "Triton
# FlashAttention"): context for the reader, not a target and not comparable
# hardware.
PAGES_CONTEXT = {
    "hardware": "NVIDIA T4 (the pages' figures; context only, not a target)",
    "best_fwd_tflops": 22.6, "best_fwd_frac_of_nominal_peak": 0.35,
    "fwd_speedup_vs_sdpa_mem_efficient": [1.55, 1.92],
    "fwdbwd_speedup_vs_sdpa_mem_efficient": [1.64, 1.83],
    "peak_extra_memory_mib": {"this_method": 130, "sdpa_mem_efficient": 226},
}


def peak_memory(torch, case, dev):
    """Peak device memory of one forward + backward through the autograd entry
    point, beyond the inputs: the four outputs (O, dQ, dK, dV) plus what the
    method keeps per query row (LSE, and the rowsum workspace)."""
    from exact_attention_88_amd.autograd import attention
    q, k, v = (dev[n].detach().clone().requires_grad_(True) for n in ("q", "k", "v"))
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    o = attention(q, k, v, causal=case.causal, scale=case.scale)
    o.backward(dev["do"])
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    rows = case.B * case.H * case.Sq
    outputs = (2 * rows + 2 * case.B * case.H * case.Sk) * case.D * q.element_size()
    del o, q, k, v
    return {"peak_beyond_inputs_bytes": int(peak), "outputs_bytes": int(outputs),
            "beyond_outputs_bytes": int(peak - outputs),
            "beyond_outputs_bytes_per_query_row": round((peak - outputs) / rows, 2),
            "materialised_fp32_scores_bytes": int(rows * case.Sk * 4)}


def library_source_sha():
    import glob
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(root, "exact_attention_88_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, scaled by the plain-copy calibration; None when the
    counters were taken on a different version of the kernel sources."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha") != library_source_sha():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else round(float(k["bytes"]))


def cpu_baseline(case, x, heads):
    """The CPU oracle, as it stands, on `heads` heads of the same workload."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    for hh in range(heads):
        h = hh % case.H
        q, k, v, do = (np.asarray(x[n][0, h]) for n in ("q", "k", "v", "do"))
        oracle.head_forward(q, k, v, case.scale, case.causal)
        oracle.head_backward(q, k, v, do, case.scale, case.causal)
    dt = time.perf_counter() - t0
    flops = 3.5 * fwd_flops(1, heads, case.Sq, case.Sk, case.D, case.causal)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"{heads} of {case.B * case.H} heads (b=0) of the same workload, forward + "
                       f"backward, float64 numpy materialised attention, {dt:.1f} s; TFLOP/s under "
                       f"the same causal accounting as the GPU figure")}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(heads would shard across GPUs with no communication)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        nbytes = 512 << 20
        src = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda").normal_()
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": 5}), flush=True)
        return
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from exact_attention_88_amd import fa
    from exact_attention_88_amd import workloads as W

    case = W.long_case()
    x, dev = make_device_inputs(case, torch)
    wall, avg = time_path(fa, torch, case, dev, args.steps, args.warmup)
    ff = fwd_flops(case.B, case.H, case.Sq, case.Sk, case.D, case.causal)
    ms_step = wall / args.steps * 1e3
    value = 3.5 * ff / (wall / args.steps) / 1e12
    fwd_tf = ff / (avg["fwd"] * 1e-3) / 1e12
    # Dominant kernel: the longest average launch.  Algorithmic flops per launch:
    # forward = 2 matmul units (QK^T, PV), dK/dV = 4 (S, dV, dP, dK), dQ = 3
    # (S, dP, dQ); one unit = 2*B*H*Sq*Sk*D flops (halved when causal).
    unit = ff / 2
    units = {"fwd": 2, "bwd_dkdv": 4, "bwd_dq": 3}
    dom = max(units, key=lambda n: avg[n])
    achieved = units[dom] * unit / (avg[dom] * 1e-3) / 1e12
    line = {
        "metric": "attention TFLOP/s fwd+bwd (fp16, causal, D=128)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: Q,K,V,dO iid N(0,1) rounded to fp16, seed 4",
        "config": {"workload": "long-context causal fp16 attention fwd+bwd, B=1 H=16 S=16384 D=128",
                   "B": case.B, "H": case.H, "S": case.Sq, "D": case.D, "causal": True},
        "fwd_tflops": round(fwd_tf, 2),
        "fwd_frac_of_peak": round(fwd_tf / MFMA_PEAK_F16, 4),
        "fwdbwd_frac_of_peak": round(value / MFMA_PEAK_F16, 4),
        "kernel_ms": {n: round(v, 4) for n, v in avg.items()},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": MFMA_PEAK_F16, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_F16, 4),
                     "traffic": measured_traffic(dom)},
    }
    if not args.no_bf16:
        # Secondary figure: the same workload in bfloat16 (inputs rounded to
        # bfloat16 from the same draws), same accounting.
        import dataclasses
        bcase = dataclasses.replace(case, name="long_bf16_causal", dtype="bf16")
        _, bdev = make_device_inputs(bcase, torch)
        bsteps = max(3, args.steps // 2)
        bwall, bavg = time_path(fa, torch, bcase, bdev, bsteps, args.warmup)
        line["bf16"] = {"fwd_tflops": round(ff / (bavg["fwd"] * 1e-3) / 1e12, 2),
                        "fwdbwd_tflops": round(3.5 * ff / (bwall / bsteps) / 1e12, 2),
                        "ms_per_step": round(bwall / bsteps * 1e3, 4), "steps": bsteps,
                        "kernel_ms": {n: round(v, 4) for n, v in bavg.items()}}
        del bdev
    line["memory"] = peak_memory(torch, case, dev)
    # Secondary ceilings: the measured MFMA rate, and the exponential rate
    # against the step's exponentials (one per visible score in the forward,
    # the dQ and the dK/dV kernels: 3 x B*H*Sq*Sk, halved when causal).
    probes = probe_rates(fa, torch)
    n_exp = 3 * case.B * case.H * case.Sq * case.Sk / (2 if case.causal else 1)
    probes["exp2_floor_ms_per_step"] = round(n_exp / probes["exp2_per_s"] * 1e3, 4)
    line["probes"] = probes
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, x, args.cpu_heads)
    if not args.no_length_sweep or args.sweep:
        del dev
        sweep = length_sweep(fa, torch, max(3, args.steps // 2), 20)
        line["length_sweep"] = sweep
        if args.sweep:
            with open(args.sweep, "w") as f:
                for rec in sweep:
                    f.write(json.dumps(rec) + "\n")
    line["context"] = PAGES_CONTEXT
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
