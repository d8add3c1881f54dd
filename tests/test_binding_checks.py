"""CPU checks of the Python binding's argument checks: every tensor's shape
and dtype is compared with q's [B, H, Sq, D] and k's Sk before anything
reaches the library, so a short or differently typed tensor is refused with
ValueError instead of being read or written past its end by a kernel.

All tensors here live in host memory: a well-formed call is refused too (the
library runs on the GPU only), so no call reaches the C ABI.
"""
import pytest

torch = pytest.importorskip("torch")
fa = pytest.importorskip("exact_attention_88_amd.fa")

B, H, SQ, SK, D = 2, 3, 5, 7, 64


def _qkv(dtype=torch.float16):
    q = torch.zeros(B, H, SQ, D, dtype=dtype)
    k = torch.zeros(B, H, SK, D, dtype=dtype)
    v = torch.zeros(B, H, SK, D, dtype=dtype)
    return q, k, v


def _rows(n=SQ, dtype=torch.float32):
    return torch.zeros(B, H, n, dtype=dtype)


def test_well_formed_host_tensors_are_refused_as_host_memory():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="GPU only"):
        fa.fa_fwd(q, k, v, True, 0.125)
    with pytest.raises(ValueError, match="GPU only"):
        fa.fa_bwd(q, k, v, q.clone(), q.clone(), _rows(), True, 0.125)


@pytest.mark.parametrize("which,shape", [
    ("k", (B, H, SK, 32)),      # head dim differs from q's
    ("k", (B, H + 1, SK, D)),   # heads differ
    ("v", (B, H, SK - 1, D)),   # v shorter than k
    ("v", (1, H, SK, D)),       # batch differs
])
def test_fwd_rejects_key_value_shapes(which, shape):
    q, k, v = _qkv()
    t = torch.zeros(shape, dtype=torch.float16)
    args = dict(q=q, k=k, v=v)
    args[which] = t
    with pytest.raises(ValueError, match="Sk, D"):
        fa.fa_fwd(args["q"], args["k"], args["v"], False, 0.125)


def test_fwd_rejects_output_shape_and_dtype():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="Sq, D"):
        fa.fa_fwd(q, k, v, False, 0.125, out=torch.zeros(B, H, SQ - 1, D, dtype=torch.float16))
    with pytest.raises(ValueError, match="dtype"):
        fa.fa_fwd(q, k, v, False, 0.125, out=torch.zeros(B, H, SQ, D, dtype=torch.float32))


@pytest.mark.parametrize("lse", [
    torch.zeros(B, H, SQ - 1),                        # short
    torch.zeros(B, H, SQ, dtype=torch.float16),       # wrong dtype
    torch.zeros(B, SQ, H).transpose(1, 2),            # not contiguous
])
def test_fwd_rejects_bad_lse(lse):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="lse"):
        fa.fa_fwd(q, k, v, False, 0.125, lse=lse)


def test_fwd_rejects_mixed_input_dtypes():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="dtype"):
        fa.fa_fwd(q, k.float(), v, False, 0.125)
    with pytest.raises(ValueError, match="dtype"):
        fa.fa_fwd(q.float(), k.float(), v, False, 0.125)


@pytest.mark.parametrize("name,shape", [
    ("o", (B, H, SQ, D + 64)),
    ("dout", (B, H, SQ + 1, D)),
    ("dq", (B, H, SK, D)),
    ("dk", (B, H, SQ, D)),
    ("dv", (B, H, SK - 2, D)),
])
def test_bwd_rejects_tensor_shapes(name, shape):
    q, k, v = _qkv()
    args = dict(o=q.clone(), dout=q.clone(), dq=None, dk=None, dv=None)
    args[name] = torch.zeros(shape, dtype=torch.float16)
    with pytest.raises(ValueError, match="expected"):
        fa.fa_bwd(q, k, v, args["o"], args["dout"], _rows(), True, 0.125, dq=args["dq"],
                  dk=args["dk"], dv=args["dv"])


@pytest.mark.parametrize("name", ["o", "dout", "dq", "dk", "dv"])
def test_bwd_rejects_tensor_dtypes(name):
    q, k, v = _qkv()
    args = dict(o=q.clone(), dout=q.clone(), dq=None, dk=None, dv=None)
    like = k if name in ("dk", "dv") else q
    args[name] = torch.zeros(like.shape, dtype=torch.float32)
    with pytest.raises(ValueError, match="dtype"):
        fa.fa_bwd(q, k, v, args["o"], args["dout"], _rows(), True, 0.125, dq=args["dq"],
                  dk=args["dk"], dv=args["dv"])


@pytest.mark.parametrize("which", ["lse", "delta"])
@pytest.mark.parametrize("bad", ["short", "dtype"])
def test_bwd_rejects_row_vectors(which, bad):
    q, k, v = _qkv()
    badt = _rows(SQ - 1) if bad == "short" else _rows(dtype=torch.float16)
    lse = badt if which == "lse" else _rows()
    delta = badt if which == "delta" else None
    with pytest.raises(ValueError, match="lse and delta"):
        fa.fa_bwd(q, k, v, q.clone(), q.clone(), lse, True, 0.125, delta=delta)


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan")])
def test_c_abi_rejects_scale_that_is_not_finite_and_positive(scale):
    """The C ABI's own check (FA_ERR_SCALE), reached through the raw library
    with never-dereferenced pointers."""
    import ctypes
    lib = fa.raw_lib()
    s = (ctypes.c_int64 * 4)(1 << 20, 1 << 16, 128, 1)
    vp = ctypes.c_void_p
    st = lib.fa_fwd(vp(0x10000), s, vp(0x20000), s, vp(0x30000), s, 1, 1, 8, 8, 64, 0,
                    ctypes.c_float(scale), 0, vp(0x40000), s, vp(0x50000), vp(0))
    assert st == -9
    st = lib.fa_bwd(vp(0x10000), s, vp(0x20000), s, vp(0x30000), s, vp(0x40000), s, vp(0x50000), s,
                    vp(0x60000), 1, 1, 8, 8, 64, 1, ctypes.c_float(scale), 0, vp(0x70000),
                    vp(0x80000), s, vp(0x90000), s, vp(0xa0000), s, vp(0))
    assert st == -9
    assert "scale" in fa.fa_status_string(-9)
