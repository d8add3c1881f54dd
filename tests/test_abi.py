"""CPU checks of the C boundary: the library loads, exports every function
that include/fa.h declares, and rejects bad arguments before any HIP call;
the same for the probe library and include/fa_probe.h.

No call here reaches a kernel launch: every call either fails validation or
is a documented no-op, so these run without a GPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
PROBE_HEADER = os.path.join(ROOT, "include", "fa_probe.h")

fa = pytest.importorskip("exact_attention_88_amd.fa")
lib = fa.raw_lib()

I64x4 = ctypes.c_int64 * 4
FAKE = 0x10000  # a non-null address that is never dereferenced by a rejected call
S = I64x4(1 << 20, 1 << 16, 128, 1)


def _declared(header=HEADER):
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", txt)))


def _exported(path):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    return set(re.findall(r"\bT (fa_[a-z_0-9]+)", out))


def test_header_declarations_match_binding():
    assert _declared() == sorted(fa.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    exported = _exported(fa.lib_path())
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_probe_library_exports_its_header_and_nothing_of_the_attention_api():
    from exact_attention_88_amd import probe
    assert _declared(PROBE_HEADER) == sorted(probe.EXPORTED_SYMBOLS)
    exported = _exported(probe.lib_path())
    for name in _declared(PROBE_HEADER):
        assert name in exported, name
    assert not exported & set(_declared())            # no attention entry point
    assert not _exported(fa.lib_path()) & set(_declared(PROBE_HEADER))  # and no probe in libfa


def test_version_and_status_strings():
    assert "gfx950" in fa.fa_version()
    for code in range(0, -11, -1):
        assert fa.fa_status_string(code).startswith("FA_")
    assert "unknown" in fa.fa_status_string(-99)


def _fwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE + 4096, lse=FAKE + 8192, B=1, H=1, Sq=8, Sk=8, D=64,
         causal=0, dtype=0, qs=S, ks=S, vs=S, os_=S, tile=None):
    args = [ctypes.c_void_p(q), qs, ctypes.c_void_p(k), ks, ctypes.c_void_p(v), vs, B, H, Sq, Sk,
            D, causal, ctypes.c_float(0.125), dtype, ctypes.c_void_p(o), os_,
            ctypes.c_void_p(lse), ctypes.c_void_p(0)]
    if tile is None:
        return lib.fa_fwd(*args)
    return lib.fa_fwd_tile(tile, *args)


def _bwd(B=1, H=1, Sq=8, Sk=8, D=64, dtype=0, ptrs=None, strides=None, tiles=None, causal=0):
    p = dict(q=FAKE, k=FAKE + 1 * 4096, v=FAKE + 2 * 4096, o=FAKE + 3 * 4096,
             do=FAKE + 4 * 4096, lse=FAKE + 5 * 4096, delta=FAKE + 6 * 4096,
             dq=FAKE + 7 * 4096, dk=FAKE + 8 * 4096, dv=FAKE + 9 * 4096)
    p.update(ptrs or {})
    st = dict(q=S, k=S, v=S, o=S, do=S, dq=S, dk=S, dv=S)
    st.update(strides or {})
    vp = ctypes.c_void_p
    args = [vp(p["q"]), st["q"], vp(p["k"]), st["k"], vp(p["v"]), st["v"], vp(p["o"]), st["o"],
            vp(p["do"]), st["do"], vp(p["lse"]), B, H, Sq, Sk, D, causal, ctypes.c_float(0.125),
            dtype, vp(p["delta"]), vp(p["dq"]), st["dq"], vp(p["dk"]), st["dk"], vp(p["dv"]),
            st["dv"], vp(0)]
    if tiles is None:
        return lib.fa_bwd(*args)
    return lib.fa_bwd_tile(tiles[0], tiles[1], *args)


def test_fwd_rejects_bad_dtype():
    assert _fwd(dtype=7) == -3


def test_causal_mode_must_be_0_1_or_2():
    assert _fwd(causal=3) == -8
    assert _fwd(causal=-1) == -8
    assert _bwd(causal=3) == -8


@pytest.mark.parametrize("D", [0, 8, 48, 96, 256])
def test_fwd_rejects_unsupported_head_dim(D):
    assert _fwd(D=D) == -2


@pytest.mark.parametrize("kw", [dict(B=-1), dict(H=-2), dict(Sq=-1), dict(Sk=-5),
                                dict(Sk=0), dict(Sq=1 << 31), dict(B=1 << 20, H=1 << 12)])
def test_fwd_rejects_bad_sizes(kw):
    assert _fwd(**kw) == -2


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_fwd_rejects_null_pointers(name):
    assert _fwd(**{name: 0}) == -1


def test_fwd_rejects_null_stride_array():
    assert _fwd(qs=None) == -1


def test_fwd_rejects_negative_stride():
    assert _fwd(ks=I64x4(0, 0, -128, 1)) == -4


@pytest.mark.parametrize("alias", [dict(o=FAKE), dict(lse=FAKE), dict(lse=FAKE + 4096)])
def test_fwd_rejects_aliased_outputs(alias):
    assert _fwd(**alias) == -5


def test_fwd_empty_problem_is_noop_without_pointers():
    assert _fwd(q=0, k=0, v=0, o=0, lse=0, Sq=0) == 0
    assert _fwd(q=0, k=0, v=0, o=0, lse=0, B=0) == 0
    assert _fwd(q=0, k=0, v=0, o=0, lse=0, H=0, Sk=0) == 0


def test_fwd_rejects_out_of_range_tile():
    n = fa.fa_tile_count(fa.FA_PASS_FWD, 0, 64)
    assert _fwd(tile=n) == -7
    assert _fwd(tile=-2) == -7


def test_bwd_validation():
    assert _bwd(dtype=5) == -3
    assert _bwd(D=40) == -2
    assert _bwd(Sk=0) == -2
    assert _bwd(ptrs=dict(dk=0)) == -1
    assert _bwd(ptrs=dict(delta=0)) == -1
    assert _bwd(strides=dict(dv=I64x4(0, -1, 64, 1))) == -4
    assert _bwd(ptrs=dict(dq=FAKE)) == -5            # dq aliases q
    assert _bwd(ptrs=dict(dk=FAKE + 9 * 4096)) == -5  # dk aliases dv
    assert _bwd(ptrs=dict(delta=FAKE + 5 * 4096)) == -5  # delta aliases lse
    assert _bwd(B=0) == 0
    assert _bwd(Sq=0, Sk=0) == 0
    n = fa.fa_tile_count(fa.FA_PASS_BWD_DKDV, 0, 64)
    assert _bwd(tiles=(n, 0)) == -7
    m = fa.fa_tile_count(fa.FA_PASS_BWD_DQ, 0, 64)
    assert _bwd(tiles=(0, m)) == -7


@pytest.mark.parametrize("dtype", [0, 1, 2])
@pytest.mark.parametrize("D", [16, 32, 64, 128])
def test_tile_tables_fit_lds_and_are_consistent(dtype, D):
    for p in (fa.FA_PASS_FWD, fa.FA_PASS_BWD_DKDV, fa.FA_PASS_BWD_DQ):
        n = fa.fa_tile_count(p, dtype, D)
        assert n >= 1
        for t in range(n):
            bm, bn, waves, lds = fa.fa_tile_info(p, dtype, D, t)
            assert lds <= 160 * 1024
            assert bm % 32 == 0 and bn % 32 == 0 and waves in (1, 2, 4, 8)
        with pytest.raises(fa.FAError):
            fa.fa_tile_info(p, dtype, D, n)
        d = fa.fa_tile_default(p, dtype, D, 4096, 4096, True)
        assert 0 <= d < n
    assert fa.fa_tile_count(0, dtype, 48) == 0
    assert fa.fa_tile_count(9, dtype, D) == 0


def _swept_table():
    """kSweptTiles from the generated table, as a nested list."""
    import os
    import re
    path = os.path.join(os.path.dirname(fa.__file__), "csrc", "fa_tile_table.inc")
    body = re.sub(r"//[^\n]*", "", open(path).read()).split("=", 1)[1]
    nums = [int(x) for x in re.findall(r"-?\d+", body)]
    assert len(nums) == 3 * 3 * 4 * 2 * 8
    it = iter(nums)
    return [[[[[next(it) for _ in range(8)] for _ in range(2)] for _ in range(4)] for _ in range(3)]
            for _ in range(3)]


@pytest.mark.parametrize("pass_id", [0, 1, 2])
def test_tile_default_follows_the_swept_table(pass_id):
    """The default configuration is the sweep's pick for the power-of-two
    bucket of max(Sq, Sk), clamped to 128..16384 (lengths between two buckets
    take the larger one), for every dtype, head dim and causal mode."""
    table = _swept_table()
    for dtype in (0, 1, 2):
        for di, D in enumerate((16, 32, 64, 128)):
            n = fa.fa_tile_count(pass_id, dtype, D)
            for causal in (0, 1, 2):
                for bi in range(8):
                    b = 128 << bi
                    want = table[pass_id][dtype][di][1 if causal else 0][bi]
                    lens = [(b, b), (b // 2 + 1, b), (b, 7)] if bi else [(1, 1), (100, 128), (128, 3)]
                    if bi == 7:
                        lens.append((3 * b, b))  # longer than the last bucket: clamped to it
                    for Sq, Sk in lens:
                        d = fa.fa_tile_default(pass_id, dtype, D, Sq, Sk, causal)
                        assert 0 <= d < n
                        if want >= 0:
                            assert d == want, (pass_id, dtype, D, causal, Sq, Sk, d, want)


def test_probe_rejects_bad_arguments_before_any_launch():
    from exact_attention_88_amd import probe
    plib = probe.raw_lib()
    sink = ctypes.c_void_p(FAKE)
    assert plib.fa_probe(2, 10, sink, None) == -2     # unknown kind
    assert plib.fa_probe(-1, 10, sink, None) == -2
    assert plib.fa_probe(0, 0, sink, None) == -2      # no iterations
    assert plib.fa_probe(1, 10, None, None) == -1     # no sink


def _bwd_noalloc(B=1, H=1, Sq=8, Sk=8, D=64, dtype=0, causal=0, scale=0.125, ptrs=None):
    p = dict(q=FAKE, k=FAKE + 1 * 4096, v=FAKE + 2 * 4096, o=FAKE + 3 * 4096,
             do=FAKE + 4 * 4096, lse=FAKE + 5 * 4096, dq=FAKE + 7 * 4096, dk=FAKE + 8 * 4096,
             dv=FAKE + 9 * 4096)
    p.update(ptrs or {})
    vp = ctypes.c_void_p
    return lib.fa_bwd_noalloc(vp(p["q"]), S, vp(p["k"]), S, vp(p["v"]), S, vp(p["o"]), S,
                              vp(p["do"]), S, vp(p["lse"]), B, H, Sq, Sk, D, causal,
                              ctypes.c_float(scale), dtype, vp(p["dq"]), S, vp(p["dk"]), S,
                              vp(p["dv"]), S, vp(0))


def test_bwd_noalloc_validation_before_any_hip_call():
    """The allocation-free backward checks what fa_bwd checks, and its scratch
    limit (B*H*Sq <= 2^22), before touching the device."""
    assert _bwd_noalloc(B=1, H=16, Sq=(1 << 18) + 1) == -10   # one row past the scratch
    assert _bwd_noalloc(B=1 << 10, H=1 << 10, Sq=8) == -10
    assert _bwd_noalloc(dtype=9) == -3
    assert _bwd_noalloc(D=40) == -2
    assert _bwd_noalloc(scale=0.0) == -9
    assert _bwd_noalloc(causal=5) == -8
    assert _bwd_noalloc(ptrs=dict(dq=0)) == -1
    assert _bwd_noalloc(ptrs=dict(dk=FAKE)) == -5          # dk aliases q
    assert _bwd_noalloc(B=0) == 0
    assert _bwd_noalloc(Sq=0, Sk=0) == 0
    assert "scratch" in fa.fa_status_string(-10)
