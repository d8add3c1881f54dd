"""GPU parity: the HIP library (through the C ABI) against the CPU float64 oracle.

Small and mid sizes are compared element by element; the long-context and
length-sweep workloads are compared on sampled rows that the oracle computes
one by one (each sampled row uses its full score row or column).  Outputs are
NaN-poisoned before each call, so a comparison also proves that every element
was written.
"""
import numpy as np
import pytest

from exact_attention_88_amd import workloads as W
from tests import devutil as U

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _fa():
    from exact_attention_88_amd import fa
    return fa


def run_case(case, tiles=(-1, -1, -1), layout_out=None, x=None):
    """Run fa_fwd + fa_bwd for a workload case (inputs from the case's seeded
    generator unless ``x`` is given); returns the inputs and host results."""
    fa = _fa()
    x = W.make_inputs(case) if x is None else x
    tdt = U.torch_dtype(case.dtype)
    dq_t = {n: U.to_device(a, dtype=tdt) for n, a in x.items()}
    lay = layout_out or case.layout
    B, H, Sq, Sk, D = case.B, case.H, case.Sq, case.Sk, case.D
    o = U.empty_like_layout((B, H, Sq, D), tdt, lay)
    lse = U.nan_vec((B, H, Sq))
    print(f"[gpu] fwd {case.name} tiles={tiles}", flush=True)
    fa.fa_fwd_tile(tiles[0], dq_t["q"], dq_t["k"], dq_t["v"], case.causal, case.scale, out=o,
                   lse=lse)
    dq = U.empty_like_layout((B, H, Sq, D), tdt, lay)
    dk = U.empty_like_layout((B, H, Sk, D), tdt, lay)
    dv = U.empty_like_layout((B, H, Sk, D), tdt, lay)
    delta = U.nan_vec((B, H, Sq))
    print(f"[gpu] bwd {case.name} tiles={tiles}", flush=True)
    fa.fa_bwd_tile(tiles[1], tiles[2], dq_t["q"], dq_t["k"], dq_t["v"], o, dq_t["do"], lse,
                   case.causal, case.scale, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    return x, {n: U.host(t) for n, t in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv,
                                              delta=delta).items()}


def check_full(case, x, got):
    import oracle
    o, lse = oracle.attention_forward(x["q"], x["k"], x["v"], case.scale, case.causal)
    dq, dk, dv = oracle.attention_backward(x["q"], x["k"], x["v"], x["do"], case.scale,
                                           case.causal)
    ref = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
    errs = {}
    for name, r in ref.items():
        assert not np.isnan(got[name]).any(), f"{case.name}: {name} has unwritten (NaN) elements"
        errs[name] = U.err(got[name], r, case.dtype, name)
    # delta is rowsum(dO o O) of the device's own O
    dref = oracle.delta_rowsum(x["do"], got["o"])
    errs["delta"] = float(np.max(np.abs(got["delta"] - dref)) / max(1.0, np.max(np.abs(dref))))
    print(f"[parity] {case.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    for name in ref:
        assert errs[name] <= U.tol(case.dtype, name), (case.name, name, errs[name])
    assert errs["delta"] <= U.delta_tol(case.dtype)
    return errs


def test_tiny_f32_noncausal():
    case = W.tiny_case()
    x, got = run_case(case)
    check_full(case, x, got)


def test_mid_f16_causal():
    case = W.mid_case()
    x, got = run_case(case)
    check_full(case, x, got)


@pytest.mark.parametrize("case", W.edge_cases(), ids=lambda c: c.name)
def test_edge_shapes(case):
    x, got = run_case(case)
    check_full(case, x, got)


EXTRA = [
    W.Case("ragged_nonsquare_f16", 2, 3, 37, 53, 32, "f16", False, seed=101),
    W.Case("ragged_nonsquare_f32", 2, 3, 37, 53, 32, "f32", False, seed=102),
    W.Case("causal_sq_gt_sk_f16", 1, 2, 100, 37, 64, "f16", True, seed=103),
    W.Case("causal_sq_lt_sk_f16", 1, 2, 37, 100, 64, "f16", True, seed=104),
    W.Case("causal_sq_lt_sk_f32", 1, 2, 45, 130, 128, "f32", True, seed=105),
    W.Case("single_row_f16", 1, 1, 1, 1, 64, "f16", True, seed=106),
    W.Case("single_query_many_keys_f32", 2, 1, 1, 300, 16, "f32", False, seed=107),
    W.Case("many_queries_one_key_f16", 1, 2, 300, 1, 128, "f16", False, seed=108),
    W.Case("page3_shape_200x96_f32", 1, 1, 200, 96, 128, "f32", False, seed=109),
    W.Case("page3_shape_100_f16_causal", 2, 1, 100, 100, 64, "f16", True, seed=110),
]


@pytest.mark.parametrize("case", EXTRA, ids=lambda c: c.name)
def test_extra_shapes(case):
    x, got = run_case(case)
    check_full(case, x, got)


def _rising_inputs(case, growth):
    """Keys scaled up along the sequence, so that every query row's running
    maximum rises many times while the keys stream past (the online-softmax
    rescale path, taken whenever a tile raises a row maximum)."""
    x = W.make_inputs(case)
    ramp = (1.0 + growth * np.arange(case.Sk) / max(1, case.Sk - 1)).astype(np.float64)
    k = x["k"].astype(np.float64) * ramp[None, None, :, None]
    x["k"] = W.round_to_bf16(k.astype(np.float32)) if case.dtype == "bf16" else k.astype(x["k"].dtype)
    return x


RISING = [(dname, D, causal, t) for dname, D in (("f16", 128), ("bf16", 128), ("f16", 64),
                                                 ("bf16", 64), ("f32", 64))
          for causal in (False, True)
          for t in range(5 if D == 128 and dname != "f32" else 2 if dname != "f32" else 1)]


@pytest.mark.parametrize("dname,D,causal,t", RISING,
                         ids=[f"{d}-D{D}-{'c' if c else 'nc'}-t{t}" for d, D, c, t in RISING])
def test_rising_scores_rescale(dname, D, causal, t):
    """Scores grow along the keys (running maxima rise by far more than the
    forward's lazy-rescale threshold over the sequence); every tuned 16-bit
    forward variant (the first five entries at D=128, two at D=64) is forced
    in turn."""
    case = W.Case(f"rising_{dname}_D{D}_{causal}", 1, 2, 700, 700, D, dname, causal,
                  seed=300 + D, q_mult=4.0)
    fa = _fa()
    nf = fa.fa_tile_count(fa.FA_PASS_FWD, {"f16": 0, "f32": 1, "bf16": 2}[dname], D)
    x, got = run_case(case, tiles=(t % nf, -1, -1), x=_rising_inputs(case, 3.0))
    check_full(case, x, got)


BOTTOM_RIGHT = [
    W.Case("br_sq_lt_sk_f16_D64", 1, 2, 100, 300, 64, "f16", 2, seed=500),
    W.Case("br_sq_lt_sk_f16_D128", 1, 2, 200, 700, 128, "f16", 2, seed=501, layout="bshd"),
    W.Case("br_sq_lt_sk_f32_D32", 2, 2, 37, 90, 32, "f32", 2, seed=502),
    W.Case("br_sq_lt_sk_bf16_D128", 1, 2, 300, 1000, 128, "bf16", 2, seed=503),
    W.Case("br_sq_gt_sk_f16_D64", 1, 2, 300, 100, 64, "f16", 2, seed=504),
    W.Case("br_sq_gt_sk_f16_D128", 1, 2, 700, 200, 128, "f16", 2, seed=505, layout="bshd"),
    W.Case("br_sq_gt_sk_f32_D16", 2, 2, 90, 37, 16, "f32", 2, seed=506),
    W.Case("br_sq_gt_sk_bf16_D128", 1, 2, 1000, 333, 128, "bf16", 2, seed=507),
    W.Case("br_sq_eq_sk_f16_D128", 1, 2, 333, 333, 128, "f16", 2, seed=508),
    W.Case("br_one_key_f16_D128", 1, 2, 77, 1, 128, "f16", 2, seed=509),
]


def _random_cases(n=24, seed=1234):
    """Seeded random shapes over every supported axis at once: batch, heads,
    ragged Sq and Sk (1..700, independent), head dim, dtype, mask (none,
    top-left, bottom-right) and storage layout."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        D = int(rng.choice([16, 32, 64, 128]))
        dname = str(rng.choice(["f16", "bf16", "f32"]))
        causal = int(rng.integers(0, 3))
        Sq, Sk = int(rng.integers(1, 701)), int(rng.integers(1, 701))
        if causal == 1:
            Sk = max(Sk, Sq)  # top-left causal: every query row sees key 0
        layout = str(rng.choice(["bhsd", "bshd"]))
        out.append(W.Case(f"rand{i}_{dname}_D{D}_c{causal}_{Sq}x{Sk}_{layout}",
                          int(rng.integers(1, 3)), int(rng.integers(1, 4)), Sq, Sk, D, dname, causal,
                          seed=1000 + i, layout=layout))
    return out


@pytest.mark.parametrize("case", _random_cases(), ids=lambda c: c.name)
def test_random_shapes(case):
    """Seeded random shapes, compared element by element with the oracle."""
    x, got = run_case(case)
    check_full(case, x, got)


@pytest.mark.parametrize("case", BOTTOM_RIGHT, ids=lambda c: c.name)
def test_bottom_right_causal(case):
    """causal = 2: query i sees keys j <= i + Sk - Sq; rows with no visible key
    give O = 0, LSE = -inf and no gradient."""
    x, got = run_case(case)
    check_full(case, x, got)
    if case.Sq > case.Sk:
        n = case.Sq - case.Sk
        assert np.all(got["o"][:, :, :n] == 0) and np.all(np.isneginf(got["lse"][:, :, :n]))
        assert np.all(got["dq"][:, :, :n] == 0)


@pytest.mark.parametrize("case", W.bf16_cases(), ids=lambda c: c.name)
def test_bf16_cases(case):
    x, got = run_case(case)
    check_full(case, x, got)


def test_contiguous_outputs_from_strided_inputs():
    case = W.edge_cases()[2]
    x, got = run_case(case, layout_out="bhsd")
    check_full(case, x, got)


def _in_layout(a, layout, tdt):
    """Device copy of a logical [B,H,S,D] host array stored as ``layout``:
    "bhsd" contiguous, "bshd" a transposed view (row stride H*D), "pad" rows
    of D + 64 elements of which the first D are used."""
    B, H, S, D = a.shape
    t = torch.from_numpy(np.ascontiguousarray(a)).to(tdt).cuda()
    if layout == "bhsd":
        return t
    if layout == "bshd":
        store = torch.empty((B, S, H, D), dtype=tdt, device="cuda").transpose(1, 2)
    else:
        store = torch.empty((B, H, S, D + 64), dtype=tdt, device="cuda")[..., :D]
    store.copy_(t)
    return store


MIXED = [
    W.Case("mixed_layouts_f16_causal", 2, 3, 777, 777, 128, "f16", 1, seed=811),
    W.Case("mixed_layouts_f16", 2, 3, 777, 777, 128, "f16", 0, seed=812),
    W.Case("mixed_layouts_bf16_causal", 2, 3, 777, 777, 128, "bf16", 1, seed=813),
    W.Case("mixed_layouts_f16_bottom_right", 2, 3, 333, 901, 128, "f16", 2, seed=814),
]


@pytest.mark.parametrize("case", MIXED, ids=lambda c: c.name)
def test_buffer_load_kernels_with_a_layout_per_operand(case):
    """The buffer-load kernels (forward tile 4, dK/dV tile 4, dQ tile 5 of the
    16-bit D = 128 lists) compute each operand's per-lane byte offsets from
    that operand's own row stride: here Q is contiguous, K and dO are
    transposed views, V and O have padded rows, dK and dV are transposed
    views; ragged lengths (777 = 3*256 + 9 = 6*128 + 9) and, in one case,
    Sq != Sk with bottom-right masking."""
    fa = _fa()
    x = W.make_inputs(case)
    tdt = U.torch_dtype(case.dtype)
    lay = dict(q="bhsd", k="bshd", v="pad", do="bshd")
    dev = {n: _in_layout(a, lay[n], tdt) for n, a in x.items()}
    B, H, Sq, Sk, D = case.B, case.H, case.Sq, case.Sk, case.D
    o = _in_layout(np.full((B, H, Sq, D), np.nan, np.float32), "pad", tdt)
    lse = U.nan_vec((B, H, Sq))
    assert dev["k"].stride(2) != dev["v"].stride(2) != dev["q"].stride(2)
    assert o.stride(2) != dev["do"].stride(2)
    print(f"[gpu] fwd {case.name}", flush=True)
    fa.fa_fwd_tile(4, dev["q"], dev["k"], dev["v"], case.causal, case.scale, out=o, lse=lse)
    dq = U.empty_like_layout((B, H, Sq, D), tdt, "bhsd")
    dk = U.empty_like_layout((B, H, Sk, D), tdt, "bshd")
    dv = U.empty_like_layout((B, H, Sk, D), tdt, "bshd")
    delta = U.nan_vec((B, H, Sq))
    print(f"[gpu] bwd {case.name}", flush=True)
    fa.fa_bwd_tile(4, 5, dev["q"], dev["k"], dev["v"], o, dev["do"], lse, case.causal,
                   case.scale, dq=dq, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    got = {n: U.host(t) for n, t in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv,
                                          delta=delta).items()}
    check_full(case, x, got)


MANY_HEADS = [
    W.Case("many_heads_f16_causal", 8, 8, 300, 300, 128, "f16", 1, seed=821),
    W.Case("many_heads_bf16_causal", 4, 16, 300, 300, 128, "bf16", 1, seed=822),
    W.Case("many_heads_f16_bottom_right", 8, 8, 200, 300, 128, "f16", 2, seed=823),
]


@pytest.mark.parametrize("case", MANY_HEADS, ids=lambda c: c.name)
def test_causal_block_order_across_heads(case):
    """64 (b,h) pairs: every XCD holds 8 whole heads, so the causal kernels
    hand out their blocks rank by rank across those heads (largest first);
    every output element is still written once and matches the oracle."""
    x, got = run_case(case)
    check_full(case, x, got)


def test_no_queries_gives_zero_key_gradients():
    fa = _fa()
    k = torch.randn(1, 2, 40, 64, device="cuda", dtype=torch.float16)
    v = torch.randn_like(k)
    q = torch.empty(1, 2, 0, 64, device="cuda", dtype=torch.float16)
    o = torch.empty_like(q)
    lse = torch.empty(1, 2, 0, device="cuda")
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    fa.fa_bwd(q, k, v, o, o.clone(), lse, True, 0.125, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0


@pytest.mark.parametrize("dq_tile", [-1, 0], ids=["dq-default", "dq-generic"])
def test_stages_in_order_reproduce_fa_bwd(dq_tile):
    """Stages 0, 2, 1 run one by one give fa_bwd_tile's results bitwise, both
    where the dQ kernel forms delta itself (16-bit D = 128 default) and where
    the rowsum kernel does (a forced generic dQ tile); and the two paths agree
    with each other within the fp16 tolerances."""
    fa = _fa()
    case = W.Case("stages_f16", 2, 2, 300, 300, 128, "f16", True, seed=112)
    x = W.make_inputs(case)
    d = {n: U.to_device(a, dtype=torch.float16) for n, a in x.items()}
    o, lse = fa.fa_fwd(d["q"], d["k"], d["v"], True, case.scale)
    outs = []
    for staged in (False, True):
        dq, dk, dv = (torch.full_like(d["q"], float("nan")) for _ in range(3))
        delta = torch.full_like(lse, float("nan"))
        if staged:
            for stage in (0, 2, 1):
                fa.fa_bwd_stage(stage, dq_tile if stage != 1 else -1, d["q"], d["k"], d["v"], o,
                                d["do"], lse, True, case.scale, dq=dq, dk=dk, dv=dv, delta=delta)
        else:
            fa.fa_bwd_tile(-1, dq_tile, d["q"], d["k"], d["v"], o, d["do"], lse, True, case.scale,
                           dq=dq, dk=dk, dv=dv, delta=delta)
        torch.cuda.synchronize()
        outs.append([U.host(t) for t in (dq, dk, dv, delta)])
    for a, b in zip(*outs):
        assert not np.isnan(a).any()
        assert np.array_equal(a, b)
    if dq_tile == -1:
        ref = [U.host(t) for t in fa.fa_bwd_tile(-1, 0, d["q"], d["k"], d["v"], o, d["do"], lse,
                                                  True, case.scale)]
        torch.cuda.synchronize()
        for name, a, r in zip(("dq", "dk", "dv"), outs[0][:3], ref[:3]):
            assert np.max(np.abs(a - r)) / np.max(np.abs(r)) <= 2e-3, name
        assert np.max(np.abs(outs[0][3] - ref[3])) <= 1e-3 * max(1.0, np.max(np.abs(ref[3])))


def test_deterministic_bitwise():
    case = W.Case("det_f16", 2, 2, 513, 513, 128, "f16", True, seed=111)
    _, a = run_case(case)
    _, b = run_case(case)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def _tile_cases():
    fa = _fa()
    out = []
    for dtype, dname in ((0, "f16"), (1, "f32"), (2, "bf16")):
        for D in (16, 32, 64, 128):
            nf = fa.fa_tile_count(fa.FA_PASS_FWD, dtype, D)
            nkv = fa.fa_tile_count(fa.FA_PASS_BWD_DKDV, dtype, D)
            nq = fa.fa_tile_count(fa.FA_PASS_BWD_DQ, dtype, D)
            for t in range(max(nf, nkv, nq)):
                out.append((dname, D, (t % nf, t % nkv, t % nq)))
    return out


try:
    TILE_CASES = _tile_cases()
except Exception:  # library not built: collected tests will fail loudly in run_case
    TILE_CASES = []


@pytest.mark.parametrize("dname,D,tiles", TILE_CASES,
                         ids=[f"{d}-D{D}-t{t}" for d, D, t in TILE_CASES])
@pytest.mark.parametrize("causal", [False, True])
def test_every_tile_configuration(dname, D, tiles, causal):
    """Every tile-table entry, forced, on ragged shapes (square when causal)."""
    Sq, Sk = (333, 333) if causal else (200, 333)
    case = W.Case(f"tiles_{dname}_D{D}_{tiles}_{causal}", 1, 2, Sq, Sk, D, dname, causal,
                  seed=200 + D)
    x, got = run_case(case, tiles=tiles)
    check_full(case, x, got)


@pytest.mark.parametrize("dname,D,tiles", TILE_CASES,
                         ids=[f"{d}-D{D}-t{t}" for d, D, t in TILE_CASES])
@pytest.mark.parametrize("shape", [(200, 333), (333, 200)], ids=["sq<sk", "sq>sk"])
def test_every_tile_configuration_bottom_right(dname, D, tiles, shape):
    Sq, Sk = shape
    case = W.Case(f"tiles_br_{dname}_D{D}_{tiles}_{Sq}x{Sk}", 1, 2, Sq, Sk, D, dname, 2,
                  seed=600 + D)
    x, got = run_case(case, tiles=tiles)
    check_full(case, x, got)


# ------------------------------------------------------------- full sizes, sampled

def _sample_rows(S, rng, n=96):
    rows = set(range(min(32, S))) | set(range(max(0, S - 32), S))
    rows |= set(rng.choice(S, size=min(n, S), replace=False).tolist())
    return np.array(sorted(rows))


def _all_heads(case):
    return [(b, h) for b in range(case.B) for h in range(case.H)]


def _spread_heads(case, n):
    """n (b, h) pairs spread evenly over the B*H heads (first and last included)."""
    hs = _all_heads(case)
    idx = sorted({round(i * (len(hs) - 1) / max(1, n - 1)) for i in range(n)})
    return [hs[i] for i in idx]


def check_sampled(case, x, got, kheads, seed=0, nrows=96):
    """Sampled rows against the oracle.  Every head: O, LSE, dQ and delta at
    the first and last 32 query rows plus ``nrows`` random ones (each with its
    full score row).  The heads in ``kheads``: dK and dV at sampled key rows
    too (each needs every query row's LSE and softmax term, the costly part).
    Heads run in a thread pool, BLAS one thread per worker."""
    import concurrent.futures as cf
    import os
    import oracle
    from threadpoolctl import threadpool_limits
    kset = set(kheads)

    def one(bh):
        b, h = bh
        rng = np.random.default_rng((seed, b, h))
        qr = _sample_rows(case.Sq, rng, nrows)
        q, k, v, do = (x[n][b, h] for n in ("q", "k", "v", "do"))
        o_ref, l_ref = oracle.head_forward_rows(q, k, v, case.scale, case.causal, qr)
        errs = dict(o=U.err(got["o"][b, h][qr], o_ref, case.dtype, "o"),
                    lse=U.err(got["lse"][b, h][qr], l_ref, case.dtype, "lse"))
        if bh in kset:
            kr = _sample_rows(case.Sk, rng, nrows)
            dq_ref, dk_ref, dv_ref = oracle.head_backward_rows(q, k, v, do, case.scale,
                                                               case.causal, qr, kr)
            errs["dk"] = U.err(got["dk"][b, h][kr], dk_ref, case.dtype, "dk")
            errs["dv"] = U.err(got["dv"][b, h][kr], dv_ref, case.dtype, "dv")
        else:
            dq_ref = oracle.head_backward_qrows(q, k, v, do, case.scale, case.causal, qr)
        errs["dq"] = U.err(got["dq"][b, h][qr], dq_ref, case.dtype, "dq")
        dref = oracle.delta_rowsum(do[qr], got["o"][b, h][qr])
        errs["delta"] = float(np.max(np.abs(got["delta"][b, h][qr] - dref)) /
                              max(1.0, np.max(np.abs(dref))))
        return bh, errs

    workers = max(1, min(16, os.cpu_count() or 1))
    worst = {}
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(one, _all_heads(case)))
    for (b, h), errs in results:
        for name, e in errs.items():
            worst[name] = max(worst.get(name, 0.0), e)
            bar = U.delta_tol(case.dtype) if name == "delta" else U.tol(case.dtype, name)
            assert e <= bar, (case.name, b, h, name, e)
    print(f"[parity-sampled] {case.name} {len(results)} heads ({len(kset)} with key rows), "
          "worst: " + " ".join(f"{k}={v:.2e}" for k, v in sorted(worst.items())), flush=True)
    for name in ("o", "lse", "dq", "dk", "dv", "delta"):
        assert not np.isnan(got[name]).any(), f"{case.name}: {name} has NaN"
    return worst


@pytest.mark.slow
def test_long_context_sampled():
    case = W.long_case()
    x, got = run_case(case)
    check_sampled(case, x, got, _spread_heads(case, 4))


@pytest.mark.slow
def test_long_context_bf16_sampled():
    """The long workload in bfloat16 (the bench's second figure): the same
    draws rounded to bfloat16, sampled rows against the oracle."""
    import dataclasses
    case = dataclasses.replace(W.long_case(), name="long_bf16_causal", dtype="bf16")
    x, got = run_case(case)
    check_sampled(case, x, got, _spread_heads(case, 4), seed=1)


@pytest.mark.slow
@pytest.mark.parametrize("dname,causal", [("f16", True), ("f16", False), ("bf16", True)])
def test_long_context_d64_sampled(dname, causal):
    """Head dim 64 at the long workload's size (B=1, H=16, S=16384): the tuned
    D=64 forward, dQ and dK/dV kernels over many tiles and every XCD, sampled
    rows against the oracle."""
    case = W.Case(f"long_d64_{dname}_{'c' if causal else 'nc'}", 1, 16, 16384, 16384, 64, dname,
                  causal, seed=80 + (2 if dname == "bf16" else 0) + int(causal))
    x, got = run_case(case)
    check_sampled(case, x, got, _spread_heads(case, 2), seed=2)


@pytest.mark.slow
@pytest.mark.parametrize("case", W.sweep_cases(), ids=lambda c: c.name)
def test_length_sweep_sampled(case):
    x, got = run_case(case)
    check_sampled(case, x, got, _spread_heads(case, 2 if case.Sq >= 8192 else 4))


@pytest.mark.slow
@pytest.mark.parametrize("D", [128, 64])
def test_wide_row_stride_takes_the_64bit_path(D):
    """Rows 64 Ki elements apart (a [S, 512, 128] store seen one head at a
    time, its first D columns): byte offsets of the last key rows pass 2^31,
    beyond the 32-bit offsets of the buffer-load kernels, so the library must
    run kernels with 64-bit addressing (register-staged at D = 128, the
    generic ones at D = 64); sampled rows against the oracle."""
    fa = _fa()
    S, stride = 16640, 512 * 128
    case = W.Case(f"wide_stride_f16_causal_D{D}", 1, 1, S, S, D, "f16", True, seed=71)
    assert (S + 3 * 64) * stride * 2 >= 1 << 31  # past every kernel's 31-bit limit
    x = W.make_inputs(case)
    dev = {}
    for n, a in x.items():
        store = torch.empty((S, 512, 128), dtype=torch.float16, device="cuda")
        store[:, 3, :D] = torch.from_numpy(np.ascontiguousarray(a[0, 0])).cuda()
        dev[n] = store[:, 3, :D].unsqueeze(0).unsqueeze(0)  # [1, 1, S, D], row stride 65536
        assert dev[n].stride(2) == stride
    o = torch.full((1, 1, S, D), float("nan"), dtype=torch.float16, device="cuda")
    lse = U.nan_vec((1, 1, S))
    print(f"[gpu] fwd {case.name}", flush=True)
    fa.fa_fwd(dev["q"], dev["k"], dev["v"], True, case.scale, out=o, lse=lse)
    dq, dk, dv = (torch.full_like(o, float("nan")) for _ in range(3))
    delta = U.nan_vec((1, 1, S))
    print(f"[gpu] bwd {case.name}", flush=True)
    fa.fa_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, True, case.scale, dq=dq, dk=dk,
              dv=dv, delta=delta)
    torch.cuda.synchronize()
    got = {n: U.host(t) for n, t in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv,
                                          delta=delta).items()}
    check_sampled(case, x, got, [(0, 0)])
