"""Python binding of the measurement probes in ``include/fa_probe.h``
(``libfa_probe.so``, a library of its own beside the attention library):
the device's sustained dense fp16 MFMA rate and v_exp_f32 rate, the two
ceilings the attention kernels are measured against.  Argument marshalling
only; there is no fallback if the library is missing.
"""
from __future__ import annotations

import ctypes
import os

from . import fa  # loads torch's HIP runtime and libfa.so first

__all__ = ["fa_probe", "fa_probe_threads", "lib_path", "raw_lib", "EXPORTED_SYMBOLS"]

EXPORTED_SYMBOLS = ("fa_probe", "fa_probe_threads")

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libfa_probe.so")


def _load():
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m exact_attention_88_amd.build`")
    lib = ctypes.CDLL(path)
    lib.fa_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_probe.restype = ctypes.c_int
    lib.fa_probe_threads.argtypes = []
    lib.fa_probe_threads.restype = ctypes.c_int64
    return lib


_lib = _load()


def raw_lib():
    """The ctypes handle of libfa_probe.so (for tests of the raw C ABI)."""
    return _lib


def fa_probe_threads() -> int:
    return int(_lib.fa_probe_threads())


def fa_probe(kind, iters, sink):
    """Launch a measurement probe (0 = fp16 MFMA, 1 = v_exp_f32) writing one
    float per thread to ``sink`` (float32, at least fa_probe_threads()
    elements, on the GPU) on torch's current stream; see ``fa_probe`` in
    include/fa_probe.h."""
    import torch
    if not sink.is_cuda or sink.dtype != torch.float32 or sink.numel() < fa_probe_threads():
        raise ValueError("sink must be a float32 device tensor of fa_probe_threads() elements")
    st = _lib.fa_probe(int(kind), int(iters), ctypes.c_void_p(sink.data_ptr()),
                       ctypes.c_void_p(torch.cuda.current_stream(sink.device).cuda_stream))
    if st != 0:
        raise fa.FAError(st)
