"""Python binding of the C ABI in ``include/fa.h`` (argument marshalling only).

The functions carry the C names.  They take torch tensors in logical
``[B, H, S, D]`` order with any non-negative strides, pass their device
pointers, element strides and the current HIP stream to ``libfa.so``, and
return the outputs.  Every step of the computation runs in the library's HIP
kernels; torch only allocates device memory and supplies the stream.  There is
no fallback: if ``libfa.so`` is missing or was built without the symbols,
importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["FAError", "fa_fwd", "fa_bwd", "fa_fwd_tile", "fa_bwd_tile", "fa_bwd_stage",
           "fa_bwd_noalloc",
           "fa_tile_count",
           "fa_tile_info", "fa_tile_default", "fa_status_string", "fa_last_hip_error", "fa_version",
           "lib_path",
           "FA_F16", "FA_F32", "FA_BF16", "FA_PASS_FWD", "FA_PASS_BWD_DKDV", "FA_PASS_BWD_DQ",
           "CAUSAL_NONE", "CAUSAL_TOP_LEFT", "CAUSAL_BOTTOM_RIGHT", "EXPORTED_SYMBOLS"]

FA_F16, FA_F32, FA_BF16 = 0, 1, 2
FA_PASS_FWD, FA_PASS_BWD_DKDV, FA_PASS_BWD_DQ = 0, 1, 2

EXPORTED_SYMBOLS = ("fa_fwd", "fa_bwd", "fa_fwd_tile", "fa_bwd_tile", "fa_bwd_stage",
                    "fa_bwd_noalloc", "fa_tile_count", "fa_tile_info", "fa_tile_default",
                    "fa_status_string", "fa_last_hip_error", "fa_version")

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_HERE, "libfa.so")


def _hip_runtimes():
    """Paths of every HIP runtime library mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _load():
    # torch ships its own HIP runtime.  Loading it first lets libfa.so bind to
    # that same runtime (they share the soname), so that device memory and
    # streams from torch are valid in the library; two runtimes in one process
    # would not see each other's devices.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m exact_attention_88_amd.build`"
                          " (there is no fallback path)")
    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError(f"more than one HIP runtime is loaded ({runtimes}); import torch before "
                          "loading libfa.so")
    I64P = ctypes.POINTER(ctypes.c_int64)
    vp, i64, c_int, c_float = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    fwd_args = [vp, I64P, vp, I64P, vp, I64P, i64, i64, i64, i64, i64, c_int, c_float, c_int,
                vp, I64P, vp, vp]
    bwd_args = [vp, I64P, vp, I64P, vp, I64P, vp, I64P, vp, I64P, vp, i64, i64, i64, i64, i64,
                c_int, c_float, c_int, vp, vp, I64P, vp, I64P, vp, I64P, vp]
    lib.fa_fwd.argtypes = fwd_args
    lib.fa_fwd_tile.argtypes = [c_int] + fwd_args
    lib.fa_bwd.argtypes = bwd_args
    lib.fa_bwd_tile.argtypes = [c_int, c_int] + bwd_args
    lib.fa_bwd_stage.argtypes = [c_int, c_int] + bwd_args
    # fa_bwd without the delta workspace (argument 19 of fa_bwd).
    lib.fa_bwd_noalloc.argtypes = bwd_args[:19] + bwd_args[20:]
    for name in ("fa_fwd", "fa_fwd_tile", "fa_bwd", "fa_bwd_tile", "fa_bwd_stage",
                 "fa_bwd_noalloc"):
        getattr(lib, name).restype = c_int
    lib.fa_tile_count.argtypes = [c_int, c_int, i64]
    lib.fa_tile_count.restype = c_int
    lib.fa_tile_info.argtypes = [c_int, c_int, i64, c_int, I64P]
    lib.fa_tile_info.restype = c_int
    lib.fa_tile_default.argtypes = [c_int, c_int, i64, i64, i64, c_int]
    lib.fa_tile_default.restype = c_int
    lib.fa_status_string.argtypes = [c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = ctypes.c_char_p
    return lib


_lib = _load()


class FAError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = f"{fa_status_string(status)} (status {status})"
        if status == -6:
            msg += f": {fa_last_hip_error()}"
        super().__init__(msg)


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(int(status)).decode()


def fa_last_hip_error() -> str:
    return _lib.fa_last_hip_error().decode()


def fa_version() -> str:
    return _lib.fa_version().decode()


def fa_tile_count(pass_id: int, dtype: int, D: int) -> int:
    return int(_lib.fa_tile_count(pass_id, dtype, D))


def fa_tile_info(pass_id: int, dtype: int, D: int, tile_id: int):
    """(block_m, block_n, waves, lds_bytes) of a tile configuration."""
    buf = (ctypes.c_int64 * 4)()
    st = _lib.fa_tile_info(pass_id, dtype, D, tile_id, buf)
    if st != 0:
        raise FAError(st)
    return tuple(int(x) for x in buf)


def fa_tile_default(pass_id: int, dtype: int, D: int, Sq: int, Sk: int, causal: bool) -> int:
    st = int(_lib.fa_tile_default(pass_id, dtype, D, Sq, Sk, _causal_code(causal)))
    if st < 0:
        raise FAError(st)
    return st


# ----------------------------------------------------------------- marshalling

def _strides(t):
    return (ctypes.c_int64 * 4)(*[int(s) for s in t.stride()])


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.float32:
        return FA_F32
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; fa supports float16, bfloat16 and float32")


def _stream_ptr(t):
    import torch
    if t.is_cuda:
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)
    return ctypes.c_void_p(0)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check(st):
    if st != 0:
        raise FAError(st)


def _check_4d(*ts):
    """Every tensor handed to the kernels is a 4-d tensor in device memory on
    one GPU: a host pointer reaching a kernel would be a memory fault, not an
    error code, so it is refused here."""
    dev = None
    for t in ts:
        if t.dim() != 4:
            raise ValueError("fa expects [B, H, S, D] tensors")
        if not t.is_cuda:
            raise ValueError("fa runs on the GPU only: every tensor must be in device memory")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("fa expects all tensors on the same device")


CAUSAL_NONE, CAUSAL_TOP_LEFT, CAUSAL_BOTTOM_RIGHT = 0, 1, 2


def _causal_code(causal):
    """False/True map to 0/1 (none, top-left); the ints 0, 1, 2 and the
    strings "top_left" / "bottom_right" are passed as the C ABI's codes."""
    if isinstance(causal, str):
        return {"none": 0, "top_left": 1, "bottom_right": 2}[causal]
    if isinstance(causal, bool):
        return int(causal)
    return int(causal)


def _check_layout(q, k, v, outs_like_q=(), outs_like_k=(), rows=()):
    """Shapes and dtypes of every tensor against q's [B, H, Sq, D] and k's
    Sk, before anything reaches the library: the C ABI takes one set of sizes
    and one dtype for all tensors, so a short or differently typed tensor
    would be read or written past its end by the kernels."""
    for t in (q, k, v) + tuple(outs_like_q) + tuple(outs_like_k):
        if t.dim() != 4:
            raise ValueError("fa expects [B, H, S, D] tensors")
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if tuple(k.shape) != (B, H, Sk, D) or tuple(v.shape) != (B, H, Sk, D):
        raise ValueError(f"k and v must both be [B, H, Sk, D] = [{B}, {H}, {Sk}, {D}] "
                         f"(got {tuple(k.shape)} and {tuple(v.shape)})")
    for t in outs_like_q:
        if tuple(t.shape) != (B, H, Sq, D):
            raise ValueError(f"expected a [B, H, Sq, D] = {(B, H, Sq, D)} tensor, got {tuple(t.shape)}")
    for t in outs_like_k:
        if tuple(t.shape) != (B, H, Sk, D):
            raise ValueError(f"expected a [B, H, Sk, D] = {(B, H, Sk, D)} tensor, got {tuple(t.shape)}")
    for t in (k, v) + tuple(outs_like_q) + tuple(outs_like_k):
        if t.dtype != q.dtype:
            raise ValueError(f"every tensor must have q's dtype {q.dtype} (got {t.dtype})")
    import torch
    for t in rows:
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, H, Sq):
            raise ValueError(f"lse and delta must be contiguous float32 [B, H, Sq] = {(B, H, Sq)}")


def _check_same_device(ref, *ts):
    for t in ts:
        if not t.is_cuda or t.device != ref.device:
            raise ValueError("fa expects all tensors on the same GPU")


def fa_fwd_tile(tile_id, q, k, v, causal=False, scale=None, out=None, lse=None):
    """Forward attention with a forced tile id (-1 = table default).

    Returns ``(out, lse)``; ``out`` has q's shape and dtype, ``lse`` is
    float32 ``[B, H, Sq]`` (natural log).
    """
    import torch
    _check_layout(q, k, v, (out,) if out is not None else (), (),
                  (lse,) if lse is not None else ())
    _check_4d(q, k, v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty((B, H, Sq, D), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _check_4d(q, k, v, out)
    _check_same_device(q, lse)
    st = _lib.fa_fwd_tile(int(tile_id), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                          _strides(v), B, H, Sq, Sk, D, _causal_code(causal), float(scale),
                          _dtype_code(q), _ptr(out), _strides(out), _ptr(lse), _stream_ptr(q))
    _check(st)
    return out, lse


def fa_fwd(q, k, v, causal=False, scale=None, out=None, lse=None):
    """Forward attention: ``(out, lse)``; see ``fa_fwd`` in include/fa.h."""
    return fa_fwd_tile(-1, q, k, v, causal, scale, out, lse)


def fa_bwd_tile(dkdv_tile, dq_tile, q, k, v, o, dout, lse, causal=False, scale=None, dq=None,
                dk=None, dv=None, delta=None, _stage=None):
    """Backward attention with forced tile ids (-1 = table default).

    Returns ``(dq, dk, dv, delta)``.
    """
    import torch
    _check_layout(q, k, v, tuple(t for t in (o, dout, dq) if t is not None),
                  tuple(t for t in (dk, dv) if t is not None),
                  tuple(t for t in (lse, delta) if t is not None))
    _check_4d(q, k, v, o, dout)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if scale is None:
        scale = D ** -0.5
    if dq is None:
        dq = torch.empty((B, H, Sq, D), dtype=q.dtype, device=q.device)
    if dk is None:
        dk = torch.empty((B, H, Sk, D), dtype=k.dtype, device=k.device)
    if dv is None:
        dv = torch.empty((B, H, Sk, D), dtype=v.dtype, device=v.device)
    if delta is None:
        delta = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _check_4d(q, k, v, o, dout, dq, dk, dv)
    _check_same_device(q, lse, delta)
    args = (_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v), _ptr(o),
            _strides(o), _ptr(dout), _strides(dout), _ptr(lse), B, H, Sq, Sk, D,
            _causal_code(causal), float(scale), _dtype_code(q), _ptr(delta), _ptr(dq), _strides(dq),
            _ptr(dk), _strides(dk), _ptr(dv), _strides(dv), _stream_ptr(q))
    if _stage is None:
        st = _lib.fa_bwd_tile(int(dkdv_tile), int(dq_tile), *args)
    else:
        tile = dkdv_tile if _stage == 1 else dq_tile
        st = _lib.fa_bwd_stage(int(_stage), int(tile), *args)
    _check(st)
    return dq, dk, dv, delta


def fa_bwd(q, k, v, o, dout, lse, causal=False, scale=None, dq=None, dk=None, dv=None,
           delta=None):
    """Backward attention: ``(dq, dk, dv, delta)``; see ``fa_bwd`` in include/fa.h."""
    return fa_bwd_tile(-1, -1, q, k, v, o, dout, lse, causal, scale, dq, dk, dv, delta)


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, causal=False, scale=None):
    """``fa_bwd`` for callers that cannot allocate: the outputs ``dq``, ``dk``,
    ``dv`` are required, and delta goes to the library's fixed per-device
    scratch (B*H*Sq up to 2^22); see ``fa_bwd_noalloc`` in include/fa.h.
    Returns ``(dq, dk, dv)``."""
    _check_layout(q, k, v, (o, dout, dq), (dk, dv), (lse,))
    _check_4d(q, k, v, o, dout, dq, dk, dv)
    _check_same_device(q, lse)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    if scale is None:
        scale = D ** -0.5
    st = _lib.fa_bwd_noalloc(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                             _ptr(o), _strides(o), _ptr(dout), _strides(dout), _ptr(lse), B, H,
                             Sq, Sk, D, _causal_code(causal), float(scale), _dtype_code(q),
                             _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv),
                             _strides(dv), _stream_ptr(q))
    _check(st)
    return dq, dk, dv


def fa_bwd_stage(stage, tile_id, q, k, v, o, dout, lse, causal=False, scale=None, dq=None,
                 dk=None, dv=None, delta=None):
    """One backward kernel alone: 0 = rowsum(dO.O) (nothing where the dQ kernel
    forms it; ``tile_id`` is then the dQ tile), 2 = dQ, 1 = dK/dV.  Stages
    0, 2, 1 in that order are exactly ``fa_bwd_tile``."""
    t = (tile_id, tile_id)
    return fa_bwd_tile(t[0], t[1], q, k, v, o, dout, lse, causal, scale, dq, dk, dv, delta,
                       _stage=stage)


def raw_lib():
    """The ctypes handle (for argument-validation tests that pass raw pointers)."""
    return _lib
