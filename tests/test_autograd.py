"""The autograd entry point: same kernels as the C ABI, once differentiable,
memory linear in the sequence length."""
import numpy as np
import pytest

from exact_attention_88_amd import workloads as W
from tests import devutil as U

torch = pytest.importorskip("torch")


def test_host_tensors_are_refused():
    """No CPU fallback: host tensors never reach a kernel."""
    from exact_attention_88_amd.autograd import attention
    q = torch.zeros(1, 1, 4, 16, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        attention(q, q, q)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,causal", [("f16", True), ("bf16", False), ("f32", True)])
def test_autograd_matches_c_abi_and_oracle(dtype, causal):
    import oracle
    from exact_attention_88_amd import fa
    from exact_attention_88_amd.autograd import attention
    case = W.Case(f"autograd_{dtype}", 2, 3, 300, 300, 64, dtype, causal, seed=400,
                  layout="bshd")
    x = W.make_inputs(case)
    tdt = U.torch_dtype(dtype)
    q, k, v, do = (U.to_device(x[n], dtype=tdt) for n in ("q", "k", "v", "do"))
    q.requires_grad_(True); k.requires_grad_(True); v.requires_grad_(True)
    print(f"[gpu] autograd {case.name}", flush=True)
    o = attention(q, k, v, causal=causal, scale=case.scale)
    o.backward(do)
    torch.cuda.synchronize()
    # bitwise equal to the direct C-ABI calls
    o2, lse2 = fa.fa_fwd(q.detach(), k.detach(), v.detach(), causal, case.scale)
    dq2, dk2, dv2, _ = fa.fa_bwd(q.detach(), k.detach(), v.detach(), o2, do, lse2, causal,
                                 case.scale)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    assert torch.equal(q.grad, dq2) and torch.equal(k.grad, dk2) and torch.equal(v.grad, dv2)
    # and within tolerance of the oracle
    ro, _ = oracle.attention_forward(x["q"], x["k"], x["v"], case.scale, causal)
    rdq, rdk, rdv = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], case.scale, causal)
    for name, got, ref in (("o", o, ro), ("dq", q.grad, rdq), ("dk", k.grad, rdk),
                           ("dv", v.grad, rdv)):
        e = U.err(U.host(got), ref, dtype, name)
        assert e <= U.tol(dtype, name), (name, e)


@pytest.mark.gpu
def test_double_backward_is_refused():
    from exact_attention_88_amd.autograd import attention
    q = torch.randn(1, 2, 64, 32, device="cuda", dtype=torch.float16, requires_grad=True)
    k = torch.randn_like(q, requires_grad=True)
    v = torch.randn_like(q, requires_grad=True)
    o = attention(q, k, v, causal=True)
    (g,) = torch.autograd.grad(o.float().square().sum(), q, create_graph=True)
    with pytest.raises(RuntimeError):
        torch.autograd.grad(g.float().sum(), q)


@pytest.mark.gpu
def test_peak_extra_memory_is_linear_in_length():
    """Forward + backward through the autograd call: device memory beyond the
    inputs and the four outputs (O, dQ, dK, dV) is O(B*H*S) -- the LSE and
    the rowsum workspace, 8 bytes per query row -- never O(S^2)."""
    from exact_attention_88_amd.autograd import attention
    extra = {}
    for S in (2048, 4096):
        B, H, D = 1, 8, 128
        q, k, v, do = (torch.randn(B, H, S, D, device="cuda", dtype=torch.float16)
                       for _ in range(4))
        for t in (q, k, v):
            t.requires_grad_(True)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        o = attention(q, k, v, causal=True)
        o.backward(do)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        outputs = 4 * B * H * S * D * 2  # O, dQ, dK, dV
        extra[S] = peak - outputs
        del o, q, k, v, do
    rows = {S: 8 * S for S in extra}  # B*H*S rows
    for S, e in extra.items():
        # LSE + delta = 8 bytes per row, plus allocator rounding (< 2 MiB)
        assert e <= 8 * rows[S] + (2 << 20), (S, e)
