"""Helpers for the GPU parity tests: device tensors in the workloads' storage
layouts, NaN-poisoned outputs, and the error measures with their tolerances.

Tolerances (the pages' own ones existed only because of TF32, so the bars here
are tighter):
  float32: max |x - ref| <= 2e-5 for O and LSE, <= 1e-4 for dQ, dK, dV;
  float16: max |x - ref| / max |ref| <= 2e-3 for O and <= 1e-2 for dQ, dK, dV,
           and max |lse - ref| <= 2e-3 (LSE is float32 from float32 sums);
  bfloat16: 1.6e-2 for O (the float16 bar scaled by the ratio of the unit
           roundoffs, 2^-8 against 2^-11: the errors come from rounding P and
           the output to the 16-bit type) and 2e-2 for dQ, dK, dV, relative
           to max |ref| (roughly the float16 gradient bar scaled the same way,
           capped at the value the objective's bfloat16 row gives); LSE as
           for float16.  Measured errors sit near 4e-3 (O) and at most about
           1.1e-2 (gradients, peaked softmax).
"""
from __future__ import annotations

import numpy as np

TOL = {
    "f32": {"o": 2e-5, "lse": 2e-5, "grad": 1e-4},
    "f16": {"o": 2e-3, "lse": 2e-3, "grad": 1e-2},
    "bf16": {"o": 1.6e-2, "lse": 2e-3, "grad": 2e-2},
}


def torch_dtype(case_dtype):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16}.get(case_dtype, torch.float32)


def to_device(x, device="cuda", dtype=None):
    """numpy [B,H,S,D] (possibly a transposed view of [B,S,H,D]) -> torch view
    with the same logical shape and the same storage order on the device,
    converted to ``dtype`` if given (exact for bfloat16-valued float32 input)."""
    import torch
    if x.flags["C_CONTIGUOUS"]:
        t = torch.from_numpy(np.array(x)).to(device)
        return t if dtype is None else t.to(dtype)
    store = np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    t = torch.from_numpy(store).to(device)
    if dtype is not None:
        t = t.to(dtype)
    return t.transpose(1, 2)


def empty_like_layout(shape, dtype, layout, device="cuda", fill=float("nan")):
    """A NaN-filled output in logical [B,H,S,D] order with the given storage layout."""
    import torch
    B, H, S, D = shape
    if layout == "bhsd":
        return torch.full((B, H, S, D), fill, dtype=dtype, device=device)
    return torch.full((B, S, H, D), fill, dtype=dtype, device=device).transpose(1, 2)


def nan_vec(shape, device="cuda"):
    import torch
    return torch.full(shape, float("nan"), dtype=torch.float32, device=device)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def err(x, ref, dtype, kind):
    """Error measure for this dtype and quantity (absolute for f32 and LSE,
    relative to max |ref| for 16-bit tensors)."""
    with np.errstate(invalid="ignore"):
        diff = np.where(x == ref, 0.0, np.abs(x - ref))  # equal infinities (LSE = -inf) match
    d = float(np.max(diff)) if x.size else 0.0
    if dtype in ("f16", "bf16") and kind != "lse":
        m = float(np.max(np.abs(ref))) if ref.size else 0.0
        return d / m if m > 0 else d
    return d


def tol(dtype, kind):
    return TOL[dtype]["grad" if kind in ("dq", "dk", "dv") else kind]


def delta_tol(dtype):
    """Bar on delta = rowsum(dO o O) against the same sum over the device's own
    O, relative to max(1, max |ref|): the device accumulates in fp32."""
    return {"f32": 1e-5, "f16": 2e-3, "bf16": 1.6e-2}[dtype]
