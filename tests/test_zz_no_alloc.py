"""GPU check of the allocation-free backward (fa_bwd_noalloc): through the C
ABI it gives exactly fa_bwd's results, on two calls in a row with the second
one smaller (the scratch array keeps the first call's contents), for the
buffer-load 16-bit D = 128 path (delta formed by the dQ kernel) and a generic
path (delta from the rowsum kernel)."""
import numpy as np
import pytest

from exact_attention_88_amd import workloads as W
from tests import devutil as U

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev(case):
    x = W.make_inputs(case)
    return {n: U.to_device(a, dtype=U.torch_dtype(case.dtype)) for n, a in x.items()}


def _both(case):
    from exact_attention_88_amd import fa
    d = _dev(case)
    print(f"[gpu] no-alloc {case.name}: forward", flush=True)
    o, lse = fa.fa_fwd(d["q"], d["k"], d["v"], case.causal, case.scale)
    ref = fa.fa_bwd(d["q"], d["k"], d["v"], o, d["do"], lse, case.causal, case.scale)[:3]
    outs = [torch.full_like(t, float("nan")) for t in ref]
    print(f"[gpu] no-alloc {case.name}: fa_bwd_noalloc", flush=True)
    fa.fa_bwd_noalloc(d["q"], d["k"], d["v"], o, d["do"], lse, *outs, causal=case.causal,
                      scale=case.scale)
    torch.cuda.synchronize()
    for name, a, r in zip(("dq", "dk", "dv"), outs, ref):
        a, r = U.host(a), U.host(r)
        assert not np.isnan(a).any(), (case.name, name)
        assert np.array_equal(a, r), (case.name, name, float(np.max(np.abs(a - r))))


@pytest.mark.parametrize("first,second", [
    (W.Case("na_big_f16_c", 2, 8, 2048, 2048, 128, "f16", True, seed=901),
     W.Case("na_small_f16_c", 1, 2, 333, 333, 128, "f16", True, seed=902)),
    (W.Case("na_big_f32_nc", 2, 4, 700, 900, 64, "f32", False, seed=903),
     W.Case("na_small_bf16_br", 1, 3, 200, 450, 32, "bf16", 2, seed=904, layout="bshd")),
    (W.Case("na_big_f16_d64_c", 2, 8, 2048, 2048, 64, "f16", True, seed=905),
     W.Case("na_small_bf16_d64_nc", 1, 2, 333, 333, 64, "bf16", False, seed=906)),
], ids=["f16-d128", "generic", "d64"])
def test_noalloc_backward_matches_fa_bwd_twice(first, second):
    _both(first)
    _both(second)
