"""Pins for the CPU float64 oracle, checked against facts outside the oracle.

Each pin comes from the mathematics of attention or from an independent
implementation, never from the oracle itself:
  * a hand-worked 2x2 example (tests/golden/hand_2x2.json);
  * closed forms: Q = 0 gives the (prefix-)mean of V and LSE = log(#visible);
    a single key gives O = v0 and zero dQ, dK;
  * invariants: softmax rows sum to one, O shifts with V, sum_j dV_j = sum_i dO_i,
    sum_j dK_j = 0, key permutation equivariance, causal row 0;
  * central finite differences of <dO, O(Q, K, V)> for all three gradients;
  * pure-Python brute force of the definition on tiny inputs;
  * torch's float64 CPU attention and autograd as a second implementation;
  * the rowsum(dO o O) shortcut against the softmax Jacobian term;
  * row-blocked evaluation equal to whole-matrix evaluation.
The mutation tests at the end plant plausible mistakes in copies of the
oracle and check that these pins catch every one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_2x2.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- pin helpers
# Each takes forward/backward callables with the per-head signatures of
# oracle.head_forward / oracle.head_backward and returns an error measure.

def pin_golden(fwd, bwd):
    g = json.load(open(GOLD))
    q, k, v, do = (np.array(g[n]) for n in ("q", "k", "v", "do"))
    err = 0.0
    for causal, key in ((False, "noncausal"), (True, "causal")):
        exp = g[key]
        o, lse = fwd(q, k, v, g["scale"], causal)
        dq, dk, dv = bwd(q, k, v, do, g["scale"], causal)
        for got, name in ((o, "o"), (lse, "lse"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
            err = max(err, float(np.max(np.abs(got - np.array(exp[name])))))
    return err


def pin_zero_query(fwd, Sq=7, Sk=7, D=3, seed=0):
    """Q = 0: uniform weights over visible keys."""
    rng = _rng(seed)
    k, v = _rand(rng, Sk, D), _rand(rng, Sk, D)
    q = np.zeros((Sq, D))
    err = 0.0
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.37, causal)
        for i in range(Sq):
            n = min(i + 1, Sk) if causal else Sk
            err = max(err, float(np.max(np.abs(o[i] - v[:n].mean(axis=0)))))
            err = max(err, abs(lse[i] - math.log(n)))
    return err


def pin_single_key(fwd, bwd, Sq=5, D=4, seed=1):
    rng = _rng(seed)
    q, k, v, do = _rand(rng, Sq, D), _rand(rng, 1, D), _rand(rng, 1, D), _rand(rng, Sq, D)
    s = 0.5
    o, lse = fwd(q, k, v, s, False)
    dq, dk, dv = bwd(q, k, v, do, s, False)
    err = float(np.max(np.abs(o - v[0])))
    err = max(err, float(np.max(np.abs(lse - s * (q @ k[0])))))
    err = max(err, float(np.max(np.abs(dq))), float(np.max(np.abs(dk))))
    err = max(err, float(np.max(np.abs(dv[0] - do.sum(axis=0)))))
    return err


def pin_rows_sum_to_one(fwd, Sq=6, Sk=9, D=5, seed=2):
    rng = _rng(seed)
    q, k, v = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D)
    s = 0.8
    err = 0.0
    for causal in (False, True):
        _, lse = fwd(q, k, v, s, causal)
        for i in range(Sq):
            tot = 0.0
            for j in range(Sk):
                if causal and j > i:
                    continue
                tot += math.exp(s * float(q[i] @ k[j]) - lse[i])
            err = max(err, abs(tot - 1.0))
    return err


def pin_value_shift(fwd, Sq=6, Sk=6, D=4, seed=3):
    rng = _rng(seed)
    q, k, v = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D)
    c = _rand(rng, D)
    err = 0.0
    for causal in (False, True):
        o1, _ = fwd(q, k, v, 0.6, causal)
        o2, _ = fwd(q, k, v + c, 0.6, causal)
        err = max(err, float(np.max(np.abs(o2 - o1 - c))))
    return err


def pin_causal_row0(fwd, bwd, S=6, D=3, seed=4):
    rng = _rng(seed)
    q, k, v, do = (_rand(rng, S, D) for _ in range(4))
    o, lse = fwd(q, k, v, 0.9, True)
    dq, _, _ = bwd(q, k, v, do, 0.9, True)
    return max(float(np.max(np.abs(o[0] - v[0]))), abs(lse[0] - 0.9 * float(q[0] @ k[0])),
               float(np.max(np.abs(dq[0]))))


def pin_grad_sums(bwd, Sq=7, Sk=5, D=3, seed=5):
    rng = _rng(seed)
    q, k, v = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D)
    do = _rand(rng, Sq, D)
    err = 0.0
    for causal in (False, True):
        _, dk, dv = bwd(q, k, v, do, 0.7, causal)
        err = max(err, float(np.max(np.abs(dv.sum(axis=0) - do.sum(axis=0)))))
        err = max(err, float(np.max(np.abs(dk.sum(axis=0)))))
    return err


def _brute_forward(q, k, v, s, causal):
    Sq, Sk, D = q.shape[0], k.shape[0], v.shape[1]
    o = [[0.0] * D for _ in range(Sq)]
    lse = [0.0] * Sq
    for i in range(Sq):
        vis = [j for j in range(Sk) if not (causal and j > i)]
        sc = {j: s * sum(float(q[i, d]) * float(k[j, d]) for d in range(q.shape[1])) for j in vis}
        z = sum(math.exp(x) for x in sc.values())
        lse[i] = math.log(z)
        for d in range(D):
            o[i][d] = sum(math.exp(sc[j]) / z * float(v[j, d]) for j in vis)
    return np.array(o), np.array(lse)


def pin_brute_force(fwd, seed=6):
    rng = _rng(seed)
    err = 0.0
    for Sq, Sk, D in ((3, 3, 2), (4, 6, 3), (5, 2, 4)):
        q, k, v = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D)
        for causal in (False, True):
            o, lse = fwd(q, k, v, 0.45, causal)
            ob, lb = _brute_forward(q, k, v, 0.45, causal)
            err = max(err, float(np.max(np.abs(o - ob))), float(np.max(np.abs(lse - lb))))
    return err


def pin_finite_differences(fwd, bwd, seed=7, h=1e-6):
    """Relative error of the analytic gradients against central differences."""
    rng = _rng(seed)
    worst = 0.0
    for Sq, Sk, D, causal in ((1, 1, 2, False), (2, 2, 2, True), (3, 3, 4, True), (5, 5, 2, False),
                              (8, 8, 4, True), (3, 5, 4, False), (5, 3, 2, True)):
        q, k, v, do = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D), _rand(rng, Sq, D)
        s = 0.55

        def loss(qq, kk, vv):
            return float(np.sum(do * fwd(qq, kk, vv, s, causal)[0]))

        grads = bwd(q, k, v, do, s, causal)
        for which, (x, g) in enumerate(zip((q, k, v), grads)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                args_p = [q.copy(), k.copy(), v.copy()]
                args_m = [q.copy(), k.copy(), v.copy()]
                args_p[which][idx] += h
                args_m[which][idx] -= h
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
            scale = max(1.0, float(np.max(np.abs(num))))
            worst = max(worst, float(np.max(np.abs(num - g))) / scale)
    return worst


def pin_torch_reference(fwd, bwd, seed=8):
    """torch's float64 CPU attention (math path) and autograd, a separate implementation."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = _rng(seed)
    err = 0.0
    for Sq, Sk, D, causal in ((9, 9, 8, False), (9, 9, 8, True), (6, 11, 4, False),
                              (11, 6, 4, True), (33, 33, 16, True)):
        q, k, v, do = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D), _rand(rng, Sq, D)
        s = 0.3
        tq, tk, tv = (torch.tensor(x[None, None], requires_grad=True) for x in (q, k, v))
        to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=s)
        to.backward(torch.tensor(do[None, None]))
        sc = s * (tq.detach() @ tk.detach().transpose(-1, -2))
        if causal:
            sc = sc.masked_fill(~torch.ones(Sq, Sk, dtype=torch.bool).tril(), float("-inf"))
        tl = torch.logsumexp(sc, dim=-1)
        o, lse = fwd(q, k, v, s, causal)
        dq, dk, dv = bwd(q, k, v, do, s, causal)
        err = max(err, float(np.max(np.abs(o - to.detach().numpy()[0, 0]))),
                  float(np.max(np.abs(lse - tl.numpy()[0, 0]))),
                  float(np.max(np.abs(dq - tq.grad.numpy()[0, 0]))),
                  float(np.max(np.abs(dk - tk.grad.numpy()[0, 0]))),
                  float(np.max(np.abs(dv - tv.grad.numpy()[0, 0]))))
    return err


def pin_row_blocking(fwd_blocked, bwd_blocked, seed=9):
    """Evaluating 3 query rows at a time equals the whole-matrix evaluation."""
    rng = _rng(seed)
    q, k, v, do = (_rand(rng, 10, 4) for _ in range(4))
    err = 0.0
    for causal in (False, True):
        o1, l1 = fwd_blocked(q, k, v, 0.5, causal, row_block=3)
        o2, l2 = _brute_forward(q, k, v, 0.5, causal)
        g1 = bwd_blocked(q, k, v, do, 0.5, causal, row_block=3)
        g2 = bwd_blocked(q, k, v, do, 0.5, causal, row_block=1000)
        err = max(err, float(np.max(np.abs(o1 - o2))), float(np.max(np.abs(l1 - l2))))
        err = max(err, max(float(np.max(np.abs(a - b))) for a, b in zip(g1, g2)))
    return err


ALL_FWD_PINS = [pin_zero_query, pin_rows_sum_to_one, pin_value_shift, pin_brute_force]
ALL_PAIR_PINS = [pin_golden, pin_single_key, pin_causal_row0, pin_finite_differences,
                 pin_torch_reference]


# ---------------------------------------------------------------- the oracle passes

def test_golden_hand_example():
    assert pin_golden(oracle.head_forward, oracle.head_backward) < 1e-12


def test_zero_query_closed_form():
    assert pin_zero_query(oracle.head_forward) < 1e-12


def test_single_key_closed_form():
    assert pin_single_key(oracle.head_forward, oracle.head_backward) < 1e-12


def test_softmax_rows_sum_to_one():
    assert pin_rows_sum_to_one(oracle.head_forward) < 1e-12


def test_value_shift_invariance():
    assert pin_value_shift(oracle.head_forward) < 1e-12


def test_causal_row_zero():
    assert pin_causal_row0(oracle.head_forward, oracle.head_backward) < 1e-12


def test_gradient_sum_invariants():
    assert pin_grad_sums(oracle.head_backward) < 1e-12


def test_brute_force_tiny():
    assert pin_brute_force(oracle.head_forward) < 1e-12


def test_finite_differences():
    assert pin_finite_differences(oracle.head_forward, oracle.head_backward) < 1e-7


def test_torch_float64_reference():
    assert pin_torch_reference(oracle.head_forward, oracle.head_backward) < 1e-12


def test_row_blocking():
    assert pin_row_blocking(oracle.head_forward, oracle.head_backward) < 1e-12


def test_key_permutation_equivariance():
    rng = _rng(10)
    q, k, v = _rand(rng, 5, 3), _rand(rng, 8, 3), _rand(rng, 8, 3)
    perm = rng.permutation(8)
    o1, l1 = oracle.head_forward(q, k, v, 0.4, False)
    o2, l2 = oracle.head_forward(q, k[perm], v[perm], 0.4, False)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_delta_shortcut_matches_softmax_term():
    """rowsum(dO o O) equals sum_j P_ij dP_ij, computed here by brute force."""
    rng = _rng(11)
    for causal in (False, True):
        q, k, v, do = (_rand(rng, 6, 3) for _ in range(4))
        o, lse = oracle.head_forward(q, k, v, 0.7, causal)
        d1 = oracle.delta_rowsum(do, o)
        for i in range(6):
            tot = 0.0
            for j in range(6):
                if causal and j > i:
                    continue
                p = math.exp(0.7 * float(q[i] @ k[j]) - lse[i])
                tot += p * float(do[i] @ v[j])
            assert abs(d1[i] - tot) < 1e-12


def test_batched_wrappers_match_heads():
    rng = _rng(12)
    q, k, v, do = (_rand(rng, 2, 3, 5, 4) for _ in range(4))
    o, lse = oracle.attention_forward(q, k, v, 0.5, True)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.5, True)
    for b in range(2):
        for h in range(3):
            oh, lh = oracle.head_forward(q[b, h], k[b, h], v[b, h], 0.5, True)
            gh = oracle.head_backward(q[b, h], k[b, h], v[b, h], do[b, h], 0.5, True)
            assert np.array_equal(o[b, h], oh) and np.array_equal(lse[b, h], lh)
            for a, g in zip((dq, dk, dv), gh):
                assert np.array_equal(a[b, h], g)


def test_float16_inputs_widen_exactly():
    """fp16 inputs are widened to float64 exactly before any arithmetic."""
    rng = _rng(13)
    q, k, v = (_rand(rng, 4, 8).astype(np.float16) for _ in range(3))
    o1, l1 = oracle.head_forward(q, k, v, 0.25, True)
    o2, l2 = oracle.head_forward(q.astype(np.float64), k.astype(np.float64),
                                 v.astype(np.float64), 0.25, True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- planted mistakes
# Copies of the oracle with one plausible mistake each; at least one pin must fail.

def _mut_forward(kind):
    def fwd(q, k, v, scale, causal, row_block=A.ROW_BLOCK):
        q, k, v = A._f64(q), A._f64(k), A._f64(v)
        Sq = q.shape[0]
        o = np.empty((Sq, v.shape[1]))
        lse = np.empty(Sq)
        for r0 in range(0, Sq, row_block):
            r1 = min(Sq, r0 + row_block)
            s = (scale if kind != "no_scale" else 1.0) * (q[r0:r1] @ k.T)
            if causal:
                off = 0 if kind == "mask_offset" else r0
                rows = np.arange(off, off + r1 - r0)[:, None]
                cols = np.arange(k.shape[0])[None, :]
                bad = (cols < rows) if kind == "mask_flip" else (cols >= rows if kind == "mask_diag" else cols > rows)
                s = np.where(bad, -np.inf, s)
            m = s.max(axis=1, keepdims=True)
            L = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
            if kind == "lse_no_max":
                L = np.log(np.exp(s - m).sum(axis=1, keepdims=True))
            p = np.exp(s - L)
            if kind == "v_transposed":
                o[r0:r1] = (p @ v[:, ::-1])
            else:
                o[r0:r1] = p @ v
            lse[r0:r1] = L[:, 0]
        return o, lse
    return fwd


def _mut_backward(kind):
    def bwd(q, k, v, do, scale, causal, row_block=A.ROW_BLOCK):
        q, k, v, do = A._f64(q), A._f64(k), A._f64(v), A._f64(do)
        Sq = q.shape[0]
        dq = np.empty_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        for r0 in range(0, Sq, row_block):
            r1 = min(Sq, r0 + row_block)
            s = A._scores(q[r0:r1], k, scale, causal, r0)
            p = np.exp(s - A._lse(s))
            dv += p.T @ do[r0:r1]
            dp = do[r0:r1] @ v.T
            if kind == "ds_sign":
                ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))
            elif kind == "ds_no_delta":
                ds = p * dp
            else:
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[r0:r1] = (1.0 if kind == "dq_no_scale" else scale) * (ds @ k)
            if kind == "dk_uses_p":
                dk += scale * (p.T @ q[r0:r1])
            else:
                dk += scale * (ds.T @ q[r0:r1])
            if kind == "dv_uses_ds":
                dv += ds.T @ do[r0:r1] - p.T @ do[r0:r1]
        return dq, dk, dv
    return bwd


def _any_pin_fails(fwd, bwd, tol=1e-7):
    def fwd_nb(q, k, v, s, c):
        return fwd(q, k, v, s, c)

    def bwd_nb(q, k, v, do, s, c):
        return bwd(q, k, v, do, s, c)
    for pin in ALL_FWD_PINS:
        if pin(fwd_nb) > tol:
            return True
    for pin in ALL_PAIR_PINS:
        if pin(fwd_nb, bwd_nb) > tol:
            return True
    if pin_grad_sums(bwd_nb) > tol:
        return True
    if pin_row_blocking(fwd, bwd) > tol:
        return True
    return False


@pytest.mark.parametrize("kind", ["no_scale", "mask_flip", "mask_diag", "mask_offset",
                                  "lse_no_max", "v_transposed"])
def test_planted_forward_mistake_is_caught(kind):
    assert _any_pin_fails(_mut_forward(kind), oracle.head_backward)


@pytest.mark.parametrize("kind", ["ds_sign", "ds_no_delta", "dq_no_scale", "dk_uses_p",
                                  "dv_uses_ds"])
def test_planted_backward_mistake_is_caught(kind):
    assert _any_pin_fails(oracle.head_forward, _mut_backward(kind))


def test_sampled_rows_match_full_evaluation():
    """The sampled-row forms used at full sizes agree with whole-head evaluation."""
    rng = _rng(14)
    for causal in (False, True):
        q, k, v, do = _rand(rng, 37, 5), _rand(rng, 37, 5), _rand(rng, 37, 5), _rand(rng, 37, 5)
        o, lse = oracle.head_forward(q, k, v, 0.4, causal)
        dq, dk, dv = oracle.head_backward(q, k, v, do, 0.4, causal)
        rows = [0, 5, 17, 36]
        o2, l2 = oracle.head_forward_rows(q, k, v, 0.4, causal, rows)
        assert np.max(np.abs(o2 - o[rows])) < 1e-12 and np.max(np.abs(l2 - lse[rows])) < 1e-12
        krows = [1, 9, 36]
        dq2, dk2, dv2 = oracle.head_backward_rows(q, k, v, do, 0.4, causal, rows, krows,
                                                  row_block=8)
        assert np.max(np.abs(dq2 - dq[rows])) < 1e-12
        assert np.max(np.abs(dk2 - dk[krows])) < 1e-12
        assert np.max(np.abs(dv2 - dv[krows])) < 1e-12


def test_query_rows_backward_matches_full_evaluation():
    """dq of sampled query rows alone (no key-side work) equals whole-head
    evaluation, top-left and bottom-right causal and not, Sq != Sk."""
    rng = _rng(15)
    for causal, Sq, Sk in ((False, 37, 29), (True, 37, 37), (2, 23, 41), (2, 41, 23)):
        q, do = _rand(rng, Sq, 6), _rand(rng, Sq, 6)
        k, v = _rand(rng, Sk, 6), _rand(rng, Sk, 6)
        dq, _, _ = oracle.head_backward(q, k, v, do, 0.35, causal)
        rows = [0, 3, Sq // 2, Sq - 1]
        dq2 = oracle.head_backward_qrows(q, k, v, do, 0.35, causal, rows)
        assert np.max(np.abs(dq2 - dq[rows])) < 1e-12
