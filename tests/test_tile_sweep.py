"""CPU checks of the tile-sweep tool's host side: choosing the fastest entry
per cell, writing the C table, and merging runs (no GPU, no timing)."""
import json

from exact_attention_88_amd import tile_sweep as TS
from tests.test_abi import _swept_table


def _parse(path):
    import re
    body = re.sub(r"//[^\n]*", "", open(path).read()).split("=", 1)[1]
    return [int(x) for x in re.findall(r"-?\d+", body)]


def test_write_table_picks_fastest_and_marks_missing(tmp_path):
    res = {("fwd", 0, 64, 1, 4096): [0.5, 0.2, 0.3],        # fastest: 1
           ("dkdv", 2, 128, 0, 128): [0.1, 0.4],             # fastest: 0
           ("dq", 1, 16, 1, 16384): [0.9, 0.8, 0.7, 0.95]}   # fastest: 2
    out = tmp_path / "t.inc"
    TS.write_table(res, str(out), "test device")
    nums = _parse(out)
    assert len(nums) == 3 * 3 * 4 * 2 * 8

    def at(p, dt, di, c, bi):
        return nums[((((p * 3 + dt) * 4 + di) * 2 + c) * 8) + bi]

    assert at(0, 0, 2, 1, 5) == 1      # fwd fp16 D=64 causal S=4096
    assert at(1, 2, 3, 0, 0) == 0      # dkdv bf16 D=128 non-causal S=128
    assert at(2, 1, 0, 1, 7) == 2      # dq fp32 D=16 causal S=16384
    assert sum(1 for x in nums if x != -1) == 3
    assert "test device" in open(out).read()


def test_merge_later_runs_win(tmp_path):
    a = [{"pass": "fwd", "dtype": 0, "D": 128, "causal": 0, "S": 1024, "ms": [1.0, 2.0]}]
    b = [{"pass": "fwd", "dtype": 0, "D": 128, "causal": 0, "S": 1024, "ms": [3.0, 2.0]},
         {"pass": "dq", "dtype": 1, "D": 32, "causal": 1, "S": 256, "ms": [5.0, 4.0, 6.0]}]
    pa, pb, out = tmp_path / "a.json", tmp_path / "b.json", tmp_path / "m.inc"
    pa.write_text(json.dumps(a))
    pb.write_text(json.dumps(b))
    TS.main(["--out", str(out), "--merge", str(pa), str(pb), "--device", "x"])
    nums = _parse(out)
    assert nums[((((0 * 3 + 0) * 4 + 3) * 2 + 0) * 8) + 3] == 1   # b's timing replaced a's
    assert nums[((((2 * 3 + 1) * 4 + 1) * 2 + 1) * 8) + 1] == 1


def test_committed_table_is_complete():
    """Every cell of the compiled-in table was measured."""
    t = _swept_table()
    assert all(x >= 0 for p in t for d in p for h in d for c in h for x in c)


def test_dq_entries_are_timed_with_the_rowsum_stage_they_need():
    """The sweep times dQ entry t as stage 0 then stage 2 with the same tile
    (stage 0 launches the rowsum kernel only where tile t does not form the
    rowsum itself), and --passes restricts the passes swept.  Run on the CPU
    with stand-ins for the GPU calls that record them."""
    import types

    import torch

    calls = []

    class Event:
        def __init__(self, enable_timing=False):
            pass

        def record(self):
            pass

        def synchronize(self):
            pass

        def elapsed_time(self, other):
            return 1.0

    fake_torch = types.SimpleNamespace(
        Generator=lambda device=None: torch.Generator(),
        randn=lambda shape, generator=None, device=None, dtype=None: torch.randn(
            shape, generator=generator, dtype=dtype),
        empty_like=torch.empty_like, float16=torch.float16, float32=torch.float32,
        bfloat16=torch.bfloat16,
        cuda=types.SimpleNamespace(Event=Event, synchronize=lambda: None,
                                   empty_cache=lambda: None))

    class FA:
        def fa_fwd(self, q, k, v, causal):
            return torch.empty_like(q), torch.empty(q.shape[:3])

        def fa_tile_count(self, p, code, D):
            return 3

        def fa_fwd_tile(self, t, *a, **k):
            calls.append(("fwd", t))

        def fa_bwd_stage(self, stage, t, *a, **k):
            calls.append((stage, t))

    res = TS.sweep(fake_torch, FA(), rounds=1, min_ms=0.0, dtypes=["f16"], dims=[16],
                   buckets=[128], passes=["dq"], log=lambda m: None)
    assert sorted(res) == [("dq", 0, 16, c, 128) for c in (0, 1)]
    timed = [c for c in calls if c != (0, -1)]  # (0, -1): the delta set-up per causal flag
    assert timed and all(c[0] != "fwd" and c[0] != 1 for c in timed)
    assert len(timed) % 2 == 0
    for a, b in zip(timed[::2], timed[1::2]):
        assert a[0] == 0 and b[0] == 2 and a[1] == b[1], (a, b)
