#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X.

One step = the whole path over one batch of resident synthetic inputs:
fa_fwd (forward kernel) followed by the backward kernels (dQ, which forms
rowsum(dO.O) itself on this path, then dK/dV), each launched through the C ABI
on torch's current stream.

Default workload: long-context causal fp16 attention, B=1, H=16,
S=16384, D=128, Q/K/V/dO iid N(0,1) rounded to fp16.

Timing protocol ("FlashAttention-2 from PyTorch to Triton", benchmark harness
paragraph: warm-up, an L2 flush between runs, the median reported; "Triton
FlashAttention", walls list: median timers and accuracy checked at every
length): W untimed warm-up steps, then K steps, each preceded (outside its
timed region) by a 512 MiB device write that evicts L2 and the 256 MB MALL;
every step is bracketed by HIP events on the stream the kernels run on, and
the reported figures are medians over the K steps.  The wall time of the K
steps (flushes included) is reported beside them.

FLOP accounting: forward = 4*B*H*Sq*Sk*D, halved when causal ("FlashAttention-2
from PyTorch to Triton", the benchmark harness's flop count); forward+backward
= 3.5x forward (backward counted as 2.5x forward).  The roofline object
reports the dominant kernel against the dense fp16 MFMA peak of MI355X.

Beside the headline figure the line carries: the toolchain and device it ran
on, the tile configurations used, the shader clock and board power sampled
while the timed steps ran, the same step in bfloat16, the peak memory beyond
the inputs of one autograd forward + backward, the measured dense fp16 MFMA
and v_exp_f32 rates of the device, the length sweep (S = 512 ... 16384 with
B = 16384/S, causal and not, forward and forward+backward TFLOP/s and
fraction of peak), and -- in the CPU-baseline leg -- the CPU oracle timed on
the host's cores and the sampled-row parity errors of every benchmarked
length against it.

Prints ONE JSON line.  ``--gpus`` above 1 is refused: this build runs on one
GPU only (attention heads shard across GPUs with no communication).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import threading
import time

MFMA_PEAK_F16 = 2516.6  # TFLOP/s, dense fp16, MI355X (256 CU x 4096 flop/clk x 2.4 GHz)
FLUSH_BYTES = 512 << 20  # > L2 (8 x 4 MB) + MALL (256 MB)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # About half a second of untimed steps: the GPU needs that long under this
    # load to reach its working clock (the median over the timed steps also
    # discards a few slow first steps).
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg (oracle timing and the per-length parity check)")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads of the workload the CPU oracle times (default: one per worker)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device-to-device copy (for scaling HBM counters)")
    ap.add_argument("--no-length-sweep", action="store_true",
                    help="skip the fp16 length sweep (S = 512 ... 16384, causal and not)")
    ap.add_argument("--sweep", default="",
                    help="optional path: also write the length sweep's records there, one JSON line each")
    ap.add_argument("--no-bf16", action="store_true",
                    help="skip the secondary bfloat16 timing of the same workload")
    ap.add_argument("--no-d64", action="store_true",
                    help="skip the secondary head-dim-64 timing of the same workload")
    ap.add_argument("--no-flush", action="store_true",
                    help="time back-to-back steps without the cache flush (for comparison only)")
    ap.add_argument("--seq", type=int, default=0,
                    help="time the length-sweep workload at this S (fp16 causal, H=16, D=128, "
                         "B=16384/S) in place of the long-context one (for per-length profiles)")
    ap.add_argument("--head-dim", type=int, default=128, choices=(16, 32, 64, 128),
                    help="time the workload at this head dim in place of 128 (for per-head-dim "
                         "profiles; the line then names that head dim)")
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


# ----------------------------------------------------------------- environment

def environment(fa, torch):
    """Toolchain and device of this run (compiler versions are part of the
    result: "Triton FlashAttention", takeaways)."""
    rocm = ""
    for p in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            with open(p) as f:
                rocm = f.read().strip()
                break
        except OSError:
            pass
    props = torch.cuda.get_device_properties(0)
    return {
        # name, HIP version and the compiler that built the library
        "library": fa.fa_version(),
        "library_source_sha": library_source_sha(),
        "rocm": rocm,
        "torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None),
        "device": props.name, "arch": getattr(props, "gcnArchName", ""),
        "compute_units": props.multi_processor_count,
        "memory_gib": round(props.total_memory / 2**30, 1),
        "pci_bus_id": _pci_bus_id(torch),
    }


def _pci_bus_id(torch):
    """PCI address of device 0 as the HIP runtime reports it (to find its sysfs node)."""
    import ctypes
    try:
        lib = ctypes.CDLL("libamdhip64.so.7")  # torch's runtime, already mapped
        buf = ctypes.create_string_buffer(64)
        if lib.hipDeviceGetPCIBusId(buf, 64, torch.cuda.current_device()) == 0:
            return buf.value.decode().lower()
    except Exception:
        pass
    return None


class Sensors:
    """Shader clock and board power of the benchmarked GPU from its sysfs node
    (hwmon freq1_input in Hz, or the DPM level marked current in pp_dpm_sclk;
    hwmon power1_average or power1_input in microwatts), sampled by a
    background thread while a timed region runs.  Records what the box
    exposes and says so when it exposes nothing."""

    def __init__(self, pci):
        self.files = {}
        self.source = "none"
        self.samples = []
        self._stop = None
        base = None
        if pci:
            for cand in (f"/sys/bus/pci/devices/{pci}", f"/sys/bus/pci/devices/0000:{pci}"):
                if os.path.isdir(cand):
                    base = cand
                    break
        if base is None:  # fall back to the only amdgpu node, if there is exactly one
            import glob
            nodes = [d for d in glob.glob("/sys/class/drm/card*/device")
                     if os.path.exists(os.path.join(d, "pp_dpm_sclk"))]
            if len(set(os.path.realpath(d) for d in nodes)) == 1:
                base = nodes[0]
        if base is None:
            return
        import glob
        for hw in sorted(glob.glob(os.path.join(base, "hwmon", "hwmon*"))):
            for key, names in (("sclk_mhz", ("freq1_input",)),
                               ("power_w", ("power1_average", "power1_input"))):
                for n in names:
                    p = os.path.join(hw, n)
                    if key not in self.files and os.access(p, os.R_OK):
                        self.files[key] = p
        p = os.path.join(base, "pp_dpm_sclk")
        if os.access(p, os.R_OK):
            self.files["dpm_sclk"] = p
        self.source = base

    def read(self):
        out = {}
        for key, p in self.files.items():
            try:
                with open(p) as f:
                    txt = f.read()
            except OSError:
                continue
            if key == "sclk_mhz":
                out[key] = int(txt.strip()) / 1e6
            elif key == "power_w":
                out[key] = int(txt.strip()) / 1e6
            else:  # the DPM level marked current, e.g. "1: 1896Mhz *"
                cur = [ln for ln in txt.splitlines() if ln.strip().endswith("*")]
                if cur:
                    val = cur[0].split(":")[1].strip(" *").lower().replace("mhz", "")
                    try:
                        out["dpm_sclk_mhz"] = float(val)
                    except ValueError:
                        pass
        return out

    def start(self, period=0.005):
        self.samples = []
        if not self.files:
            return
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                self.samples.append(self.read())
                self._stop.wait(period)
        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()

    def stop(self):
        if self._stop is None:
            return self.summary()
        self._stop.set()
        self._thread.join()
        self._stop = None
        return self.summary()

    def summary(self):
        rec = {"source": self.source, "samples": len(self.samples)}
        for key in ("sclk_mhz", "dpm_sclk_mhz", "power_w"):
            vals = [s[key] for s in self.samples if key in s]
            if vals:
                rec[key] = {"min": round(min(vals), 1), "median": round(statistics.median(vals), 1),
                            "max": round(max(vals), 1)}
        return rec


def tiles_used(fa, case):
    dt = {"f16": fa.FA_F16, "bf16": fa.FA_BF16, "f32": fa.FA_F32}[case.dtype]
    out = {}
    for name, p in (("fwd", fa.FA_PASS_FWD), ("dkdv", fa.FA_PASS_BWD_DKDV), ("dq", fa.FA_PASS_BWD_DQ)):
        tid = fa.fa_tile_default(p, dt, case.D, case.Sq, case.Sk, case.causal)
        bm, bn, waves, lds = fa.fa_tile_info(p, dt, case.D, tid)
        out[name] = {"id": tid, "block_m": bm, "block_n": bn, "waves": waves, "lds_bytes": lds}
    return out


# ----------------------------------------------------------------- GPU timing

class Flusher:
    """A 512 MiB device buffer rewritten before every timed step, outside the
    timed region, so that no step finds its inputs in L2 or the MALL."""

    def __init__(self, torch, enabled=True):
        self.buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda") if enabled else None
        self.n = 0

    def __call__(self):
        if self.buf is not None:
            self.n += 1
            self.buf.fill_(self.n)


def time_path(fa, torch, case, dev, steps, warmup, flush, sensors=None, min_warm_s=0.0):
    """Time `steps` full passes twice over, interleaved.  Each pass: a cache
    flush (untimed), then the forward and the backward stages on the stream
    the kernels run on (torch's current stream).  A step's time comes from
    passes with one event before the forward and one after the last stage
    only (an event recorded between kernels costs the stream about 5 us);
    the per-kernel times from the interleaved passes with an event after
    every kernel.  Returns medians, means and the per-step list, the wall
    time of the timed loop, and the outputs of the last pass."""
    B, H, Sq, Sk, D = case.B, case.H, case.Sq, case.Sk, case.D
    q, k, v, do = dev["q"], dev["k"], dev["v"], dev["do"]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    sc = case.scale

    def step(ev=None, ends_only=False):
        if ev is not None:
            ev[0].record()
        fa.fa_fwd(q, k, v, case.causal, sc, out=o, lse=lse)
        if ev is not None and not ends_only:
            ev[1].record()
        # rowsum(dO.O) (nothing where the dQ kernel forms it), dQ, dK/dV: the
        # order fa_bwd runs them in.
        for j, stage in enumerate((0, 2, 1)):
            fa.fa_bwd_stage(stage, -1, q, k, v, o, do, lse, case.causal, sc, dq=dq, dk=dk, dv=dv,
                            delta=delta)
            if ev is not None and (not ends_only or j == 2):
                ev[2 + j].record()

    t_end = time.perf_counter() + min_warm_s
    i = 0
    while i < warmup or time.perf_counter() < t_end:
        flush()
        step()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    ends = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    if sensors is not None:
        sensors.start()
    t0 = time.perf_counter()
    for i in range(steps):
        flush()
        step(ends[i], ends_only=True)
        flush()
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sens = sensors.stop() if sensors is not None else None
    names = ("fwd", "bwd_pre", "bwd_dq", "bwd_dkdv")
    per = {n: [ev[j].elapsed_time(ev[j + 1]) for ev in evs] for j, n in enumerate(names)}
    per["step"] = [ev[0].elapsed_time(ev[4]) for ev in ends]
    per["step_with_kernel_events"] = [ev[0].elapsed_time(ev[4]) for ev in evs]
    res = {
        "median": {n: statistics.median(v) for n, v in per.items()},
        "mean": {n: sum(v) / len(v) for n, v in per.items()},
        "step_ms": per["step"],
        "wall_s": wall,
        "sensors": sens,
        "out": dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta),
    }
    return res


def sample_rows(S, seed, n):
    """Query (or key) rows for the sampled parity check: the first and last 16
    rows and n more drawn with a fixed seed."""
    import numpy as np
    rng = np.random.default_rng(seed)
    rows = set(range(min(16, S))) | set(range(max(0, S - 16), S))
    rows |= set(rng.choice(S, size=min(n, S), replace=False).tolist())
    return np.array(sorted(rows))


def grab_samples(case, out, key_heads, nrows=48):
    """Host copies of the device outputs at the rows the parity check uses:
    query rows of every head (O, LSE, dQ, delta) and key rows of `key_heads`
    (dK, dV)."""
    import numpy as np
    import torch
    qr = sample_rows(case.Sq, 7, nrows)
    kr = sample_rows(case.Sk, 8, nrows)
    dev = out["o"].device
    qi, ki = torch.as_tensor(qr, device=dev), torch.as_tensor(kr, device=dev)
    f = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    g = {"qrows": qr, "krows": kr, "key_heads": key_heads}
    for n in ("o", "dq", "lse", "delta"):
        g[n] = f(out[n].index_select(2, qi))
    for n in ("dk", "dv"):
        g[n] = {bh: f(out[n][bh[0], bh[1]].index_select(0, ki)) for bh in key_heads}
    return g


def length_sweep(fa, torch, steps, warmup, flush, keep_samples):
    """Forward and forward+backward TFLOP/s and fraction of the dense fp16
    MFMA peak at S = 512 ... 16384 (fp16, H = 16, D = 128, B = 16384/S: 16k
    tokens per call), causal and not, medians of flushed steps.  Causal and
    non-causal cases of one length share their seeded inputs."""
    from exact_attention_88_amd import workloads as W
    out, cached, samples = [], {}, []
    for sc in W.sweep_cases():
        key = (sc.Sq, sc.seed)
        if key not in cached:
            cached.clear()
            cached[key] = make_device_inputs(sc, torch)
        x, dev = cached[key]
        r = time_path(fa, torch, sc, dev, steps, warmup, flush, min_warm_s=0.3)
        med = r["median"]
        ff = fwd_flops(sc.B, sc.H, sc.Sq, sc.Sk, sc.D, sc.causal)
        fwd_tf = ff / (med["fwd"] * 1e-3) / 1e12
        fb_tf = 3.5 * ff / (med["step"] * 1e-3) / 1e12
        out.append({"S": sc.Sq, "B": sc.B, "causal": sc.causal,
                    "fwd_tflops": round(fwd_tf, 1), "fwd_frac_of_peak": round(fwd_tf / MFMA_PEAK_F16, 4),
                    "fwdbwd_tflops": round(fb_tf, 1),
                    "fwdbwd_frac_of_peak": round(fb_tf / MFMA_PEAK_F16, 4),
                    "ms_per_step": round(med["step"], 4),
                    "ms_per_step_min_max": [round(min(r["step_ms"]), 4), round(max(r["step_ms"]), 4)],
                    "kernel_ms": {n: round(v, 4) for n, v in med.items() if not n.startswith("step")},
                    "tiles": {k: v["id"] for k, v in tiles_used(fa, sc).items()}})
        if keep_samples:
            kh = [(0, 0), (sc.B - 1, sc.H - 1)] if sc.Sq < 8192 else [(sc.B - 1, sc.H - 1)]
            samples.append((sc, x, grab_samples(sc, r["out"], kh)))
        del r
    cached.clear()
    return out, samples


def probe_rates(torch):
    """Measured ceilings on this device: dense fp16 MFMA TFLOP/s and v_exp_f32
    exponentials per second (the probes of libfa_probe.so, timed with HIP
    events on the stream they run on after a warm-up launch)."""
    from exact_attention_88_amd import probe as fa
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


# ------------------------------------------------------------ CPU-baseline leg
# Everything below calls the CPU oracle (test infrastructure): the timed
# oracle baseline and the sampled-row parity check of every benchmarked
# length.  Skipped with --no-cpu-baseline.

def cpu_workers():
    """Threads for the oracle: the cores this process may run on, capped by
    the thread budget the environment sets (OMP_NUM_THREADS) and at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(16, n))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, x, heads, value_tflops_counted):
    """The CPU oracle, as it stands, on `heads` heads of the workload: its
    forward alone and its forward + backward, each head one task in a pool of
    worker threads with BLAS at one thread per worker, timed with
    time.perf_counter and extrapolated linearly to all B*H heads.  The oracle
    evaluates full, unskipped score rows whether or not the run is causal."""
    import concurrent.futures as cf
    import oracle
    from threadpoolctl import threadpool_limits
    nh = case.B * case.H
    heads = max(1, min(heads or min(8, cpu_workers()), nh))
    workers = min(cpu_workers(), heads)
    hs = [(i // case.H, i % case.H) for i in range(heads)]

    def fwd(bh):
        b, h = bh
        oracle.head_forward(x["q"][b, h], x["k"][b, h], x["v"][b, h], case.scale, case.causal)

    def fwdbwd(bh):
        b, h = bh
        q, k, v, do = (x[n][b, h] for n in ("q", "k", "v", "do"))
        oracle.head_forward(q, k, v, case.scale, case.causal)
        oracle.head_backward(q, k, v, do, case.scale, case.causal)

    t = {}
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(workers) as ex:
            for name, fn in (("fwd", fwd), ("fwdbwd", fwdbwd)):
                t0 = time.perf_counter()
                list(ex.map(fn, hs))
                t[name] = time.perf_counter() - t0
    scale_up = nh / heads
    fwd_s, fb_s = t["fwd"] * scale_up, t["fwdbwd"] * scale_up
    counted = 3.5 * fwd_flops(case.B, case.H, case.Sq, case.Sk, case.D, case.causal)
    oracle_flops = 4.0 * fwd_flops(case.B, case.H, case.Sq, case.Sk, case.D, False)
    return {
        "value": round(counted / fb_s / 1e12, 5), "unit": "TFLOP/s",
        "cores": workers, "kind": "oracle",
        "sample": (f"{heads} of {nh} heads of the same workload (float64 numpy materialised "
                   f"attention), {workers} worker threads, BLAS 1 thread each; measured "
                   f"{t['fwd']:.1f} s forward and {t['fwdbwd']:.1f} s forward+backward, "
                   + ("not extrapolated" if heads == nh else
                      f"extrapolated x{scale_up:g} to all heads") +
                   "; value = the GPU figure's counted flops (3.5x the causal-halved forward) / "
                   "the oracle's forward+backward seconds"),
        "extrapolated": heads != nh,
        "fwd_seconds": round(fwd_s, 3), "fwdbwd_seconds": round(fb_s, 3),
        "measured_heads": heads, "measured_fwd_seconds": round(t["fwd"], 3),
        "measured_fwdbwd_seconds": round(t["fwdbwd"], 3),
        "oracle_flops_fwdbwd_unskipped": oracle_flops,
        "gpu_speedup_fwdbwd": round(value_tflops_counted / (counted / fb_s / 1e12), 1),
        "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
    }


TOL = {"f16": {"o": 2e-3, "lse": 2e-3, "grad": 1e-2, "delta": 2e-3},
       "bf16": {"o": 1.6e-2, "lse": 2e-3, "grad": 2e-2, "delta": 1.6e-2}}


def parity_check(case, x, g):
    """Sampled-row errors of the device outputs against the oracle: O, LSE,
    dQ and delta at the sampled query rows of every head, dK and dV at the
    sampled key rows of g["key_heads"]; 16-bit errors relative to max |ref|
    (LSE absolute), the same bars as the parity tests."""
    import concurrent.futures as cf
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    qr, kr = g["qrows"], g["krows"]

    def rel(a, r):
        m = float(np.max(np.abs(r)))
        d = float(np.max(np.abs(a - r)))
        return d / m if m > 0 else d

    def one(bh):
        b, h = bh
        q, k, v, do = (x[n][b, h] for n in ("q", "k", "v", "do"))
        o_ref, l_ref = oracle.head_forward_rows(q, k, v, case.scale, case.causal, qr)
        e = {"o": rel(g["o"][b, h], o_ref),
             "lse": float(np.max(np.abs(g["lse"][b, h] - l_ref)))}
        dref = oracle.delta_rowsum(do[qr], g["o"][b, h])
        e["delta"] = float(np.max(np.abs(g["delta"][b, h] - dref)) / max(1.0, np.max(np.abs(dref))))
        if bh in g["key_heads"]:
            dq_ref, dk_ref, dv_ref = oracle.head_backward_rows(q, k, v, do, case.scale,
                                                               case.causal, qr, kr)
            e["dk"] = rel(g["dk"][bh], dk_ref)
            e["dv"] = rel(g["dv"][bh], dv_ref)
        else:
            dq_ref = oracle.head_backward_qrows(q, k, v, do, case.scale, case.causal, qr)
        e["dq"] = rel(g["dq"][b, h], dq_ref)
        return e

    heads = [(b, h) for b in range(case.B) for h in range(case.H)]
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(cpu_workers()) as ex:
            errs = list(ex.map(one, heads))
    worst = {n: max(e[n] for e in errs if n in e) for n in ("o", "lse", "dq", "dk", "dv", "delta")}
    tol = TOL[case.dtype]
    ok = all(worst[n] <= tol["grad" if n in ("dq", "dk", "dv") else n] for n in worst)
    rec = {n: float(f"{v:.3e}") for n, v in worst.items()}
    rec.update({"heads": len(heads), "key_heads": len(g["key_heads"]),
                "query_rows_per_head": int(len(qr)), "key_rows_per_head": int(len(kr)),
                "within_tolerance": bool(ok)})
    return rec


# ------------------------------------------------------------------------ main

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

    env = environment(fa, torch)
    sensors = Sensors(env["pci_bus_id"])
    flush = Flusher(torch, enabled=not args.no_flush)
    case = W.long_case()
    if args.seq:
        case = next(c for c in W.sweep_cases() if c.Sq == args.seq and c.causal)
    if args.head_dim != case.D:
        import dataclasses
        case = dataclasses.replace(case, name=f"{case.name}_d{args.head_dim}", D=args.head_dim)
    default_workload = not args.seq and case.D == 128
    x, dev = make_device_inputs(case, torch)
    r = time_path(fa, torch, case, dev, args.steps, args.warmup, flush, sensors)
    med, mean = r["median"], r["mean"]
    headline_samples = None
    if not args.no_cpu_baseline:
        headline_samples = grab_samples(case, r["out"], [(0, 0), (0, case.H - 1)])
    del r["out"]
    ff = fwd_flops(case.B, case.H, case.Sq, case.Sk, case.D, case.causal)
    value = 3.5 * ff / (med["step"] * 1e-3) / 1e12
    fwd_tf = ff / (med["fwd"] * 1e-3) / 1e12
    # Dominant kernel: the longest launch.  Algorithmic flops per launch:
    # forward = 2 matmul units (QK^T, PV), dK/dV = 4 (S, dV, dP, dK), dQ = 3
    # (S, dP, dQ); one unit = 2*B*H*Sq*Sk*D flops (halved when causal).  The
    # achieved rate uses the kernel's average launch duration over the timed
    # steps (the figure a rocprofv3 kernel trace of the same run averages).
    unit = ff / 2
    units = {"fwd": 2, "bwd_dkdv": 4, "bwd_dq": 3}
    dom = max(units, key=lambda n: mean[n])
    achieved = units[dom] * unit / (mean[dom] * 1e-3) / 1e12
    line = {
        "metric": f"attention TFLOP/s fwd+bwd (fp16, causal, D={case.D})",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med["step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: Q,K,V,dO iid N(0,1) rounded to fp16, seed 4",
        "config": {"workload": (f"{'long-context' if not args.seq else 'length-sweep'} causal fp16 "
                                f"attention fwd+bwd, B={case.B} H={case.H} S={case.Sq} D={case.D}"),
                   "B": case.B, "H": case.H, "S": case.Sq, "D": case.D, "causal": True},
        "timing": {"statistic": "median of per-step HIP-event times (events before the forward and "
                                "after the last backward stage only; per-kernel times from "
                                "interleaved steps with an event after every kernel)",
                   "ms_per_step_with_kernel_events": round(med["step_with_kernel_events"], 4),
                   "flush_before_each_step_bytes": 0 if args.no_flush else FLUSH_BYTES,
                   "ms_per_step_mean": round(mean["step"], 4),
                   "ms_per_step_min_max": [round(min(r["step_ms"]), 4), round(max(r["step_ms"]), 4)],
                   "timed_loop_wall_s_incl_flush": round(r["wall_s"], 4),
                   "passes_in_timed_loop": 2 * args.steps},
        "fwd_tflops": round(fwd_tf, 2),
        "fwd_frac_of_peak": round(fwd_tf / MFMA_PEAK_F16, 4),
        "fwdbwd_frac_of_peak": round(value / MFMA_PEAK_F16, 4),
        "kernel_ms": {n: round(v, 4) for n, v in med.items() if not n.startswith("step")},
        "kernel_ms_mean": {n: round(v, 4) for n, v in mean.items() if not n.startswith("step")},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": MFMA_PEAK_F16, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_F16, 4),
                     # bytes recorded for the long-context D=128 workload only
                     "traffic": measured_traffic(dom) if default_workload else None},
        "tiles": tiles_used(fa, case),
        "environment": env,
        "clock_power": {"during_timed_steps": r["sensors"]},
    }
    if not args.no_bf16:
        # Secondary figure: the same workload in bfloat16 (inputs rounded to
        # bfloat16 from the same draws), same accounting and protocol.
        import dataclasses
        bcase = dataclasses.replace(case, name="long_bf16_causal", dtype="bf16")
        _, bdev = make_device_inputs(bcase, torch)
        bsteps = max(5, args.steps // 2)
        br = time_path(fa, torch, bcase, bdev, bsteps, args.warmup, flush, min_warm_s=0.3)
        line["bf16"] = {"fwd_tflops": round(ff / (br["median"]["fwd"] * 1e-3) / 1e12, 2),
                        "fwdbwd_tflops": round(3.5 * ff / (br["median"]["step"] * 1e-3) / 1e12, 2),
                        "ms_per_step": round(br["median"]["step"], 4), "steps": bsteps,
                        "kernel_ms": {n: round(v, 4) for n, v in br["median"].items() if not n.startswith("step")}}
        del bdev, br
    if not args.no_d64:
        # Secondary figure: the same workload at head dim 64 (the mid
        # workload's head dim; fresh draws of that shape), same protocol, its
        # own flop count.
        import dataclasses
        dcase = dataclasses.replace(case, name="long_d64_causal", D=64)
        _, ddev = make_device_inputs(dcase, torch)
        dff = fwd_flops(dcase.B, dcase.H, dcase.Sq, dcase.Sk, dcase.D, dcase.causal)
        dsteps = max(5, args.steps // 2)
        dr = time_path(fa, torch, dcase, ddev, dsteps, args.warmup, flush, min_warm_s=0.3)
        line["d64"] = {"workload": f"B={dcase.B} H={dcase.H} S={dcase.Sq} D=64 causal fp16",
                       "fwd_tflops": round(dff / (dr["median"]["fwd"] * 1e-3) / 1e12, 2),
                       "fwdbwd_tflops": round(3.5 * dff / (dr["median"]["step"] * 1e-3) / 1e12, 2),
                       "ms_per_step": round(dr["median"]["step"], 4), "steps": dsteps,
                       "kernel_ms": {n: round(v, 4) for n, v in dr["median"].items() if not n.startswith("step")},
                       "tiles": tiles_used(fa, dcase)}
        del ddev, dr
    line["memory"] = peak_memory(torch, case, dev)
    # Secondary ceilings: the measured MFMA rate, and the exponential rate
    # against the step's exponentials (one per visible score in the forward,
    # the dQ and the dK/dV kernels: 3 x B*H*Sq*Sk, halved when causal).
    probes = probe_rates(torch)
    n_exp = 3 * case.B * case.H * case.Sq * case.Sk / (2 if case.causal else 1)
    probes["exp2_floor_ms_per_step"] = round(n_exp / probes["exp2_per_s"] * 1e3, 4)
    line["probes"] = probes
    sweep_samples = []
    if not args.no_length_sweep or args.sweep:
        del dev
        sweep, sweep_samples = length_sweep(fa, torch, max(10, args.steps), 20, flush,
                                            keep_samples=not args.no_cpu_baseline)
        line["length_sweep"] = sweep
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, x, args.cpu_heads, value)
        line["parity"] = parity_check(case, x, headline_samples)
        for rec, (sc, sx, g) in zip(line.get("length_sweep", []), sweep_samples):
            rec["parity"] = parity_check(sc, sx, g)
    if args.sweep and "length_sweep" in line:
        with open(args.sweep, "w") as f:
            for rec in line["length_sweep"]:
                f.write(json.dumps(rec) + "\n")
    line["context"] = PAGES_CONTEXT
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
