"""Seeded synthetic inputs for the attention workloads.

This module only draws random tensors and describes their shapes and memory
layouts.  It holds none of the attention arithmetic, so both the device path
and the CPU checker can take their inputs from it without sharing any of the
method.

Every tensor is standard-normal, drawn with ``numpy.random.default_rng(seed)``
in float32 in the order q, k, v, dO, and rounded to float16 (round to nearest
even, numpy's cast) when the case is half precision, or to the nearest
bfloat16 value (ties to even; kept in a float32 array, which holds every
bfloat16 value exactly) when the case is bfloat16.  The pages benchmark and
test on ``randn`` inputs of this kind ("FlashAttention-2 from PyTorch to
Triton", the benchmark harness and the test file), so no dataset is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

__all__ = ["Case", "make_inputs", "CONFIGS", "tiny_case", "sweep_cases", "edge_cases",
           "long_case", "mid_case", "scale_for", "round_to_bf16", "bf16_cases"]


@dataclass(frozen=True)
class Case:
    """One attention problem: shapes, dtype, masking, storage layout and seed.

    ``layout`` is the order of the *stored* array: ``"bhsd"`` is the contiguous
    logical order; ``"bshd"`` stores ``[B, S, H, D]`` and the logical
    ``[B, H, S, D]`` tensor is a strided view of it (row stride ``H*D``).
    ``q_mult`` multiplies Q (in float32, before any rounding) to make the
    softmax peaked.
    """
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    dtype: str            # "f16", "bf16" or "f32"
    causal: int           # 0/False none, 1/True top-left, 2 bottom-right aligned
    seed: int
    layout: str = "bhsd"
    q_mult: float = 1.0

    @property
    def np_dtype(self):
        """Host storage type: float16, or float32 (for f32 and for bf16 values)."""
        return np.float16 if self.dtype == "f16" else np.float32

    @property
    def scale(self) -> float:
        return scale_for(self.D)


def scale_for(D: int) -> float:
    """1/sqrt(D) rounded to float32, the value passed to the kernels."""
    return float(np.float32(1.0 / math.sqrt(D)))


def round_to_bf16(x):
    """float32 array -> float32 array of the nearest bfloat16 values (ties to
    even): the upper 16 bits of the float32 pattern after rounding the lower
    16.  Finite inputs only (these are normal draws)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(np.shape(x))


def _draw(rng, shape, dtype, mult=1.0, bf16=False):
    x = rng.standard_normal(shape, dtype=np.float32)
    if mult != 1.0:
        x = x * np.float32(mult)
    if bf16:
        return round_to_bf16(x)
    return x.astype(dtype)


def make_inputs(case: Case, with_grad: bool = True):
    """Return a dict of numpy arrays in *logical* ``[B, H, S, D]`` order.

    For ``layout == "bshd"`` the arrays are non-contiguous transposed views of
    ``[B, S, H, D]`` storage; ``np.ascontiguousarray`` recovers packed data and
    ``x.base`` the storage.  Keys: ``q``, ``k``, ``v`` and (if ``with_grad``)
    ``do``.
    """
    rng = np.random.default_rng(case.seed)
    dt = case.np_dtype
    out = {}
    names = ["q", "k", "v"] + (["do"] if with_grad else [])
    for name in names:
        S = case.Sq if name in ("q", "do") else case.Sk
        mult = case.q_mult if name == "q" else 1.0
        bf16 = case.dtype == "bf16"
        if case.layout == "bhsd":
            out[name] = _draw(rng, (case.B, case.H, S, case.D), dt, mult, bf16)
        elif case.layout == "bshd":
            store = _draw(rng, (case.B, S, case.H, case.D), dt, mult, bf16)
            out[name] = store.transpose(0, 2, 1, 3)
        else:
            raise ValueError(f"unknown layout {case.layout}")
    return out


# --- The five workload families -------------------------------------------

def tiny_case() -> Case:
    """fp32, non-causal, B=1 H=2 S=128 D=64."""
    return Case("tiny_f32", 1, 2, 128, 128, 64, "f32", False, seed=1)


def mid_case() -> Case:
    """fp16, causal, B=4 H=8 S=1024 D=64."""
    return Case("mid_f16_causal", 4, 8, 1024, 1024, 64, "f16", True, seed=2)


def edge_cases():
    """Ragged lengths, small and large head dims, strided [B,S,H,D] storage.

    D in {16, 32, 128} x S in {1000, 1537} x {f16, f32} x {causal, non-causal}
    (24 cases, seeds 30..53), plus the peaked-softmax case (Q x 8) for
    fp16/causal/D=128/S=1537 and its fp32 twin.
    """
    cases = []
    idx = 0
    for dtype in ("f16", "f32"):
        for causal in (False, True):
            for D in (16, 32, 128):
                for S in (1000, 1537):
                    cases.append(Case(f"edge_{dtype}_{'c' if causal else 'nc'}_D{D}_S{S}",
                                      2, 4, S, S, D, dtype, causal, seed=30 + idx,
                                      layout="bshd"))
                    idx += 1
    for dtype in ("f16", "f32"):
        cases.append(Case(f"edge_peaked_{dtype}_c_D128_S1537", 2, 4, 1537, 1537, 128, dtype,
                          True, seed=30 + idx, layout="bshd", q_mult=8.0))
        idx += 1
    return cases


def bf16_cases():
    """bfloat16 cases (the fp16 families' shapes): ragged strided [B,S,H,D]
    storage at D in {16, 64, 128}, causal and not, plus the peaked-softmax case
    (Q x 8) at D=128.  Seeds 60..."""
    cases = []
    idx = 0
    for causal in (False, True):
        for D, S in ((16, 1000), (64, 777), (128, 1000)):
            cases.append(Case(f"bf16_{'c' if causal else 'nc'}_D{D}_S{S}", 2, 4, S, S, D, "bf16",
                              causal, seed=60 + idx, layout="bshd"))
            idx += 1
    cases.append(Case("bf16_peaked_c_D128_S1537", 2, 4, 1537, 1537, 128, "bf16", True,
                      seed=60 + idx, layout="bshd", q_mult=8.0))
    return cases


def long_case() -> Case:
    """fp16, causal, B=1 H=16 S=16384 D=128."""
    return Case("long_f16_causal", 1, 16, 16384, 16384, 128, "f16", True, seed=4)


SWEEP_S = (512, 1024, 2048, 4096, 8192, 16384)


def sweep_cases():
    """fp16, H=16, D=128, B = 16384/S (16k tokens per call), causal and not."""
    cases = []
    for si, S in enumerate(SWEEP_S):
        for causal in (True, False):
            cases.append(Case(f"sweep_S{S}_{'c' if causal else 'nc'}", 16384 // S, 16, S, S, 128,
                              "f16", causal, seed=50 + si))
    return cases


CONFIGS = {
    "tiny": tiny_case,
    "mid": mid_case,
    "edge": edge_cases,
    "long": long_case,
    "sweep": sweep_cases,
}
