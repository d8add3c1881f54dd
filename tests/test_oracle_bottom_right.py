"""CPU pins for the oracle's bottom-right causal alignment (``causal=2``) and
its rows with no visible key.

Bottom-right alignment lets query i see keys j <= i + (Sk - Sq); when Sq > Sk
the first Sq - Sk rows see nothing and are defined to give O = 0, LSE = -inf
and no gradient.  Pinned by a pure-Python brute force, central finite
differences, torch's float64 attention with an explicit mask, the Q = 0
closed form, and the re-indexing identities with the top-left form; a planted
sign error in the offset is caught.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attention as A

BR = 2  # bottom-right causal mode


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _brute(q, k, v, s):
    Sq, Sk, D = q.shape[0], k.shape[0], v.shape[1]
    o = np.zeros((Sq, D))
    lse = np.full(Sq, -np.inf)
    for i in range(Sq):
        vis = [j for j in range(Sk) if j <= i + Sk - Sq]
        if not vis:
            continue
        sc = {j: s * sum(float(q[i, d]) * float(k[j, d]) for d in range(q.shape[1])) for j in vis}
        z = sum(math.exp(x) for x in sc.values())
        lse[i] = math.log(z)
        for d in range(D):
            o[i, d] = sum(math.exp(sc[j]) / z * float(v[j, d]) for j in vis)
    return o, lse


SHAPES = ((4, 4, 3), (3, 6, 2), (6, 3, 4), (1, 5, 2), (5, 1, 3))


def test_brute_force():
    rng = np.random.default_rng(20)
    for Sq, Sk, D in SHAPES:
        q, k, v = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D)
        o, lse = A.head_forward(q, k, v, 0.4, BR)
        ob, lb = _brute(q, k, v, 0.4)
        assert np.allclose(o, ob, atol=1e-13)
        assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
        fin = np.isfinite(lb)
        assert np.allclose(lse[fin], lb[fin], atol=1e-13)


def test_finite_differences():
    rng = np.random.default_rng(21)
    h = 1e-6
    for Sq, Sk, D in SHAPES:
        q, k, v, do = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D), _rand(rng, Sq, D)

        def loss(qq, kk, vv):
            return float(np.sum(do * A.head_forward(qq, kk, vv, 0.6, BR)[0]))

        grads = A.head_backward(q, k, v, do, 0.6, BR)
        for which, (x, g) in enumerate(zip((q, k, v), grads)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                p, m = [q.copy(), k.copy(), v.copy()], [q.copy(), k.copy(), v.copy()]
                p[which][idx] += h
                m[which][idx] -= h
                num[idx] = (loss(*p) - loss(*m)) / (2 * h)
            assert np.max(np.abs(num - g)) <= 1e-7 * max(1.0, np.max(np.abs(num))), (Sq, Sk, which)


def test_torch_reference_with_explicit_mask():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(22)
    for Sq, Sk, D in ((7, 11, 4), (9, 9, 8), (12, 5, 4)):
        q, k, v, do = _rand(rng, Sq, D), _rand(rng, Sk, D), _rand(rng, Sk, D), _rand(rng, Sq, D)
        live = slice(max(0, Sq - Sk), Sq)  # rows with at least one visible key
        nq = Sq - live.start
        tq = torch.tensor(q[live][None, None], requires_grad=True)
        tk, tv = (torch.tensor(x[None, None], requires_grad=True) for x in (k, v))
        mask = torch.ones(Sq, Sk, dtype=torch.bool).tril(diagonal=Sk - Sq)[live]
        to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.3)
        to.backward(torch.tensor(do[live][None, None]))
        sc = (0.3 * (tq.detach() @ tk.detach().transpose(-1, -2))).masked_fill(~mask, float("-inf"))
        tl = torch.logsumexp(sc, dim=-1)
        o, lse = A.head_forward(q, k, v, 0.3, BR)
        dq, dk, dv = A.head_backward(q, k, v, do, 0.3, BR)
        assert np.allclose(o[live], to.detach().numpy()[0, 0], atol=1e-12)
        assert np.allclose(lse[live], tl.numpy()[0, 0], atol=1e-12)
        assert np.allclose(dq[live], tq.grad.numpy()[0, 0], atol=1e-12)
        assert np.allclose(dk, tk.grad.numpy()[0, 0], atol=1e-12)
        assert np.allclose(dv, tv.grad.numpy()[0, 0], atol=1e-12)
        assert nq == Sq - live.start
        # rows with no visible key
        assert np.all(o[:live.start] == 0) and np.all(np.isneginf(lse[:live.start]))
        assert np.all(dq[:live.start] == 0)


def test_zero_query_closed_form():
    rng = np.random.default_rng(23)
    for Sq, Sk in ((5, 8), (8, 5), (6, 6)):
        v = _rand(rng, Sk, 3)
        o, lse = A.head_forward(np.zeros((Sq, 3)), _rand(rng, Sk, 3), v, 0.7, BR)
        for i in range(Sq):
            n = i + Sk - Sq + 1  # visible keys
            if n <= 0:
                assert np.all(o[i] == 0) and np.isneginf(lse[i])
            else:
                assert np.allclose(o[i], v[:n].mean(axis=0), atol=1e-14)
                assert abs(lse[i] - math.log(n)) < 1e-14


def test_reindexing_identities():
    """Bottom-right is the top-left form on re-indexed rows: equal when Sq = Sk;
    for Sq < Sk the last Sq rows of a square top-left problem whose extra
    leading query rows carry no output gradient; for Sq > Sk the square
    top-left problem on the last Sk queries, the other rows empty."""
    rng = np.random.default_rng(24)
    D, s = 4, 0.5
    # Sq = Sk
    q, k, v, do = (_rand(rng, 6, D) for _ in range(4))
    for a, b in zip(A.head_forward(q, k, v, s, BR), A.head_forward(q, k, v, s, True)):
        assert np.allclose(a, b, atol=1e-14)
    for a, b in zip(A.head_backward(q, k, v, do, s, BR), A.head_backward(q, k, v, do, s, True)):
        assert np.allclose(a, b, atol=1e-14)
    # Sq < Sk
    Sq, Sk = 4, 9
    q, do = _rand(rng, Sq, D), _rand(rng, Sq, D)
    k, v = _rand(rng, Sk, D), _rand(rng, Sk, D)
    qp = np.concatenate([_rand(rng, Sk - Sq, D), q])
    dop = np.concatenate([np.zeros((Sk - Sq, D)), do])
    o, lse = A.head_forward(q, k, v, s, BR)
    op, lp = A.head_forward(qp, k, v, s, True)
    assert np.allclose(o, op[Sk - Sq:], atol=1e-14) and np.allclose(lse, lp[Sk - Sq:], atol=1e-14)
    g = A.head_backward(q, k, v, do, s, BR)
    gp = A.head_backward(qp, k, v, dop, s, True)
    assert np.allclose(g[0], gp[0][Sk - Sq:], atol=1e-14)
    assert np.allclose(g[1], gp[1], atol=1e-14) and np.allclose(g[2], gp[2], atol=1e-14)
    # Sq > Sk
    Sq, Sk = 9, 4
    q, do = _rand(rng, Sq, D), _rand(rng, Sq, D)
    k, v = _rand(rng, Sk, D), _rand(rng, Sk, D)
    o, lse = A.head_forward(q, k, v, s, BR)
    o2, l2 = A.head_forward(q[Sq - Sk:], k, v, s, True)
    assert np.all(o[:Sq - Sk] == 0) and np.all(np.isneginf(lse[:Sq - Sk]))
    assert np.allclose(o[Sq - Sk:], o2, atol=1e-14) and np.allclose(lse[Sq - Sk:], l2, atol=1e-14)
    g = A.head_backward(q, k, v, do, s, BR)
    g2 = A.head_backward(q[Sq - Sk:], k, v, do[Sq - Sk:], s, True)
    assert np.all(g[0][:Sq - Sk] == 0) and np.allclose(g[0][Sq - Sk:], g2[0], atol=1e-14)
    assert np.allclose(g[1], g2[1], atol=1e-14) and np.allclose(g[2], g2[2], atol=1e-14)


def test_sampled_rows_match_full_evaluation():
    rng = np.random.default_rng(25)
    for Sq, Sk in ((13, 20), (20, 13)):
        q, do = _rand(rng, Sq, 4), _rand(rng, Sq, 4)
        k, v = _rand(rng, Sk, 4), _rand(rng, Sk, 4)
        o, lse = A.head_forward(q, k, v, 0.5, BR)
        dq, dk, dv = A.head_backward(q, k, v, do, 0.5, BR)
        qr, kr = np.array([0, 3, Sq - 1]), np.array([0, 5, Sk - 1])
        o2, l2 = A.head_forward_rows(q, k, v, 0.5, BR, qr)
        assert np.allclose(o2, o[qr], atol=1e-14)
        assert np.array_equal(np.isneginf(l2), np.isneginf(lse[qr]))
        assert np.allclose(l2[np.isfinite(l2)], lse[qr][np.isfinite(l2)], atol=1e-14)
        g = A.head_backward_rows(q, k, v, do, 0.5, BR, qr, kr)
        assert np.allclose(g[0], dq[qr], atol=1e-13)
        assert np.allclose(g[1], dk[kr], atol=1e-13) and np.allclose(g[2], dv[kr], atol=1e-13)


def test_planted_offset_sign_error_is_caught(monkeypatch):
    """A flipped alignment offset (Sq - Sk instead of Sk - Sq) fails the brute
    force, the closed form or the re-indexing pins."""
    monkeypatch.setattr(A, "causal_offset",
                        lambda causal, Sq, Sk: None if not causal else (Sq - Sk if int(causal) == 2 else 0))
    failed = 0
    for test in (test_brute_force, test_zero_query_closed_form, test_reindexing_identities):
        try:
            test()
        except AssertionError:
            failed += 1
    assert failed >= 1
