"""Measure every tile configuration and write the library's default table.

The block sizes are chosen per head dim and power-of-two length bucket by
timing every configuration that survived the on-chip-memory pruning ("Triton
FlashAttention": per-bucket autotuning with configurations that cannot fit
shared memory pruned first).  Here the tuning runs once, offline, on the
target GPU, and its result is compiled into the library as a static table:
for each pass (forward, dK/dV, dQ), dtype, head dim, causal flag and bucket
the fastest configuration's id.

    python -m exact_attention_88_amd.tile_sweep --out exact_attention_88_amd/csrc/fa_tile_table.inc

or, split over several runs (--dtypes, --dims, --buckets, each with --json)
and merged without a GPU by --merge.

Workload per bucket S: B = max(1, 16384 // S) sequences of S tokens, H = 16
heads (16k tokens per call, the shape of the length-sweep benchmark),
Sq = Sk = S, contiguous [B, H, S, D], N(0, 1) inputs.  Each configuration is
timed with HIP events over several interleaved rounds after a clock warm-up;
the median per-call time decides.  A dQ configuration is timed together with
the rowsum(dO.O) preprocess it needs: its own kernel, unless that
configuration forms the rowsum inside the dQ kernel.  Needs a GPU and the
built library.
"""
from __future__ import annotations

import argparse
import datetime
import json
import sys
import time

PASSES = ("fwd", "dkdv", "dq")
DTYPES = (("f16", 0), ("f32", 1), ("bf16", 2))  # index = the C ABI's dtype code
HEAD_DIMS = (16, 32, 64, 128)
BUCKETS = tuple(128 << i for i in range(8))  # 128 .. 16384


def _inputs(torch, dt, S, D, seed):
    B, H = max(1, 16384 // S), 16
    g = torch.Generator(device="cuda").manual_seed(seed)
    tdt = {"f16": torch.float16, "f32": torch.float32, "bf16": torch.bfloat16}[dt]
    mk = lambda: torch.randn((B, H, S, D), generator=g, device="cuda", dtype=torch.float32).to(tdt)
    return {n: mk() for n in ("q", "k", "v", "do")}


def _time(torch, fns, rounds, min_ms):
    """Median per-call milliseconds of each callable, interleaved over rounds."""
    for f in fns:
        f()
    torch.cuda.synchronize()
    reps = []
    for f in fns:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        f()
        e1.record()
        e1.synchronize()
        reps.append(max(1, min(50, int(min_ms / max(e0.elapsed_time(e1), 1e-3)) + 1)))
    times = [[] for _ in fns]
    for _ in range(rounds):
        for i, f in enumerate(fns):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps[i]):
                f()
            e1.record()
            e1.synchronize()
            times[i].append(e0.elapsed_time(e1) / reps[i])
    return [sorted(t)[len(t) // 2] for t in times]


def sweep(torch, fa, rounds=3, min_ms=2.0, dtypes=None, dims=None, buckets=None, passes=None,
          log=print):
    """{(pass, dtype code, D, causal, bucket): [ms per tile id]}."""
    res = {}
    seed = 0
    for dt, code in DTYPES:
        if dtypes and dt not in dtypes:
            continue
        for D in HEAD_DIMS:
            if dims and D not in dims:
                continue
            for S in BUCKETS:
                if buckets and S not in buckets:
                    continue
                seed += 1
                x = _inputs(torch, dt, S, D, seed)
                q, k, v, do = x["q"], x["k"], x["v"], x["do"]
                for causal in (0, 1):
                    o, lse = fa.fa_fwd(q, k, v, causal)
                    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
                    delta = torch.empty_like(lse)
                    fa.fa_bwd_stage(0, -1, q, k, v, o, do, lse, causal, dq=dq, dk=dk, dv=dv,
                                    delta=delta)
                    oo, ll = torch.empty_like(o), torch.empty_like(lse)
                    fns = {
                        "fwd": lambda t: (lambda: fa.fa_fwd_tile(t, q, k, v, causal, out=oo, lse=ll)),
                        "dkdv": lambda t: (lambda: fa.fa_bwd_stage(1, t, q, k, v, o, do, lse, causal,
                                                                    dq=dq, dk=dk, dv=dv, delta=delta)),
                        # Stage 0 with dQ tile t launches the rowsum kernel only where
                        # that tile does not form the rowsum itself.
                        "dq": lambda t: (lambda: (
                            fa.fa_bwd_stage(0, t, q, k, v, o, do, lse, causal,
                                            dq=dq, dk=dk, dv=dv, delta=delta),
                            fa.fa_bwd_stage(2, t, q, k, v, o, do, lse, causal,
                                            dq=dq, dk=dk, dv=dv, delta=delta))),
                    }
                    for pi, p in enumerate(PASSES):
                        if passes and p not in passes:
                            continue
                        n = fa.fa_tile_count(pi, code, D)
                        ms = _time(torch, [fns[p](t) for t in range(n)], rounds, min_ms)
                        res[(p, code, D, causal, S)] = ms
                        best = min(range(n), key=lambda t: ms[t])
                        log(f"[sweep] {p} {dt} D={D} causal={causal} S={S}: best {best} "
                            f"({ms[best]:.4f} ms) of {n}: " + " ".join(f"{m:.4f}" for m in ms))
                del x, q, k, v, do
                torch.cuda.empty_cache()
    return res


def write_table(res, path, device):
    """The generated C table: kSweptTiles[pass][dtype][D index][causal][bucket]."""
    def best(key):
        ms = res.get(key)
        return -1 if not ms else min(range(len(ms)), key=lambda t: ms[t])

    lines = [
        "// Fastest tile configuration per (pass, dtype, head dim, causal, length",
        "// bucket), measured by exact_attention_88_amd/tile_sweep.py:",
        "//   python -m exact_attention_88_amd.tile_sweep --out <this file>",
        f"// on {device}, {datetime.date.today().isoformat()}.  -1 = not measured (the",
        "// library then uses its built-in rule).  Generated file: edit by re-running",
        "// the sweep.",
        "// Index order: [pass: fwd, dK/dV, dQ][dtype: fp16, fp32, bf16]",
        "// [D: 16, 32, 64, 128][causal: no, yes][bucket: 128 << i, i = 0..7].",
        "static constexpr signed char kSweptTiles[3][3][4][2][8] = {",
    ]
    for p in PASSES:
        lines.append("  {  // " + p)
        for dt, code in DTYPES:
            lines.append("    {  // " + dt)
            for D in HEAD_DIMS:
                rows = []
                for causal in (0, 1):
                    ids = [best((p, code, D, causal, S)) for S in BUCKETS]
                    rows.append("{" + ", ".join(f"{i:2d}" for i in ids) + "}")
                lines.append(f"      {{{rows[0]}, {rows[1]}}},  // D = {D}")
            lines.append("    },")
        lines.append("  },")
    lines.append("};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", required=True, help="generated C table (fa_tile_table.inc)")
    ap.add_argument("--json", default="", help="optional: also write every timing here")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--min-ms", type=float, default=2.0, help="time each measurement at least this long")
    ap.add_argument("--dtypes", default="", help="comma list of f16,f32,bf16 (default all)")
    ap.add_argument("--dims", default="", help="comma list of head dims (default all)")
    ap.add_argument("--buckets", default="", help="comma list of lengths (default 128..16384)")
    ap.add_argument("--passes", default="", help="comma list of fwd,dkdv,dq (default all)")
    ap.add_argument("--merge", nargs="+", default=[],
                    help="no GPU: write --out from the --json files of earlier runs (later files win)")
    ap.add_argument("--device", default="", help="with --merge: the device the runs were made on")
    a = ap.parse_args(argv)
    if a.merge:
        res = {}
        for path in a.merge:
            with open(path) as f:
                for r in json.load(f):
                    res[(r["pass"], r["dtype"], r["D"], r["causal"], r["S"])] = r["ms"]
        write_table(res, a.out, a.device or "the device of the merged runs")
        print(f"wrote {a.out} from {len(res)} measured cells", flush=True)
        return
    import torch
    from exact_attention_88_amd import fa
    if not torch.cuda.is_available():
        sys.exit("tile_sweep needs a GPU")
    # Clock warm-up: the part takes a moment under load to reach its working clock.
    x = _inputs(torch, "f16", 4096, 128, 0)
    t0 = time.time()
    while time.time() - t0 < 1.5:
        fa.fa_fwd(x["q"], x["k"], x["v"], True)
        torch.cuda.synchronize()
    del x
    lst = lambda s, f=str: [f(v) for v in s.split(",") if v]
    res = sweep(torch, fa, a.rounds, a.min_ms, lst(a.dtypes), lst(a.dims, int), lst(a.buckets, int),
                lst(a.passes), log=lambda m: print(m, flush=True))
    props = torch.cuda.get_device_properties(0)
    write_table(res, a.out, f"{props.gcnArchName.split(':')[0]} ({torch.cuda.get_device_name(0)})")
    if a.json:
        with open(a.json, "w") as f:
            json.dump([{"pass": k[0], "dtype": k[1], "D": k[2], "causal": k[3], "S": k[4], "ms": v}
                       for k, v in res.items()], f)
    print(f"wrote {a.out}", flush=True)


if __name__ == "__main__":
    main()
