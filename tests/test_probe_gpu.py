"""GPU checks of the measurement probes: both launch, fill the whole sink
with finite values, and report positive rates."""
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("kind", [0, 1], ids=["mfma", "exp2"])
def test_probe_runs_and_fills_the_sink(kind):
    from exact_attention_88_amd import probe as fa
    n = fa.fa_probe_threads()
    assert n > 0 and n % 256 == 0
    sink = torch.full((n,), float("nan"), device="cuda")
    print(f"[gpu] probe kind={kind} threads={n}", flush=True)
    fa.fa_probe(kind, 64, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all().item()
    if kind == 1:  # every chain stays inside (0.5, 1); eight chains per thread
        assert (sink > 4.0).all().item() and (sink < 8.0).all().item()
