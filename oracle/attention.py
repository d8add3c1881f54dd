"""Plain CPU float64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

What it computes
----------------
FlashAttention-2 returns *exactly* standard scaled-dot-product attention; it
only avoids materialising the N x N score matrix ("FlashAttention-2 from
PyTorch to Triton", the opening description of the forward pass).  So the
oracle is that plain definition, written out with the full score matrix, in
float64, one (batch, head) at a time:

    S   = s * Q K^T                      (s = the float32 scale, widened)
    S_ij = -inf  for j > i + c  when causal
                                         (c = 0: top-left aligned lower
                                          triangle, the ``tril`` reference of
                                          the same page's test file; c = Sk - Sq:
                                          bottom-right aligned, ``causal=2``)
    LSE_i = log sum_j exp(S_ij)          (the per-row log-sum-exp L that the
                                          page stores for the backward)
    P   = exp(S - LSE)
    O   = P V

A row with no visible key (bottom-right alignment with Sq > Sk; the page
leaves such rows to later work) is defined to give LSE = -inf, P = 0, O = 0
and no gradient.

and its gradient, by the chain rule through the softmax (the page's backward
outline names dO, the saved L and rowsum(dO o O)):

    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
    dQ = s dS K
    dK = s dS^T Q

``delta_rowsum`` is the FlashAttention-2 shortcut rowsum(dO o O) for the
softmax term; the oracle's own backward uses the textbook sum_k P_ik dP_ik so
that the two can be checked against each other.

Query rows are independent, so long sequences are processed ``row_block``
query rows at a time (each with its full score row); for sizes up to
``row_block`` the whole matrix is formed at once.  Parity is pinned by the
CPU tests in ``tests/test_oracle.py`` (finite differences, closed forms,
invariants, a hand-worked example and torch's float64 CPU attention).
"""
from __future__ import annotations

import numpy as np

__all__ = ["attention_forward", "attention_backward", "delta_rowsum", "head_forward",
           "head_backward", "head_forward_rows", "head_backward_rows", "head_backward_qrows",
           "causal_offset"]

ROW_BLOCK = 2048


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def causal_offset(causal, Sq, Sk):
    """Key index of the last key query 0 sees (queries see keys j <= i + c):
    None when not causal, 0 for top-left alignment (causal True or 1), Sk - Sq
    for bottom-right alignment (causal == 2)."""
    if not causal:
        return None
    return Sk - Sq if int(causal) == 2 else 0


def _mask(s, q_rows, k_cols, off):
    """Apply the causal mask to s[len(q_rows), len(k_cols)] (absolute indices)."""
    if off is None:
        return s
    return np.where(np.asarray(k_cols)[None, :] > np.asarray(q_rows)[:, None] + off, -np.inf, s)


def _scores(q, k, scale, off, r0):
    """Scaled scores for query rows r0.. of one head, causal mask applied."""
    s = scale * (q @ k.T)
    return _mask(s, np.arange(r0, r0 + q.shape[0]), np.arange(k.shape[0]), off)


def _lse(s):
    """log sum_j exp(s_ij) for each row, shifted by the row max for range;
    -inf for a row whose every score is masked."""
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isneginf(m), 0.0, m)
    with np.errstate(divide="ignore"):
        return m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))


def _probs(s, L):
    """P = exp(S - LSE), and 0 on rows with no visible key."""
    with np.errstate(invalid="ignore"):
        return np.where(np.isneginf(L), 0.0, np.exp(s - L))


def head_forward(q, k, v, scale, causal, row_block=ROW_BLOCK):
    """One head: q [Sq,D], k [Sk,D], v [Sk,D] -> (o [Sq,D], lse [Sq])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Sq = q.shape[0]
    off = causal_offset(causal, Sq, k.shape[0])
    o = np.empty((Sq, v.shape[1]))
    lse = np.empty(Sq)
    for r0 in range(0, Sq, row_block):
        r1 = min(Sq, r0 + row_block)
        s = _scores(q[r0:r1], k, scale, off, r0)
        L = _lse(s)
        p = _probs(s, L)
        o[r0:r1] = p @ v
        lse[r0:r1] = L[:, 0]
    return o, lse


def head_backward(q, k, v, do, scale, causal, row_block=ROW_BLOCK):
    """One head: gradients (dq, dk, dv) of <dO, O(q, k, v)>."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Sq = q.shape[0]
    off = causal_offset(causal, Sq, k.shape[0])
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, Sq, row_block):
        r1 = min(Sq, r0 + row_block)
        s = _scores(q[r0:r1], k, scale, off, r0)
        p = _probs(s, _lse(s))
        dv += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v.T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[r0:r1] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


def attention_forward(q, k, v, scale, causal, row_block=ROW_BLOCK):
    """Batched forward over logical [B,H,S,D] arrays -> (o [B,H,Sq,D], lse [B,H,Sq])."""
    B, H, Sq, D = q.shape
    o = np.empty((B, H, Sq, v.shape[-1]))
    lse = np.empty((B, H, Sq))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h], v[b, h], scale, causal,
                                              row_block)
    return o, lse


def attention_backward(q, k, v, do, scale, causal, row_block=ROW_BLOCK):
    """Batched backward over logical [B,H,S,D] arrays -> (dq, dk, dv) in float64."""
    dq = np.empty(q.shape)
    dk = np.empty(k.shape)
    dv = np.empty(v.shape)
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = head_backward(q[b, h], k[b, h], v[b, h], do[b, h],
                                                         scale, causal, row_block)
    return dq, dk, dv


def delta_rowsum(do, o):
    """rowsum(dO o O) over the last axis, in float64 (the backward's preprocess)."""
    return (_f64(do) * _f64(o)).sum(axis=-1)


def head_forward_rows(q, k, v, scale, causal, rows):
    """Forward outputs for the given absolute query rows only (each row is the
    plain definition over its full score row): (o [len(rows), D], lse [len(rows)])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.asarray(rows, dtype=np.int64)
    off = causal_offset(causal, q.shape[0], k.shape[0])
    s = _mask(scale * (q[rows] @ k.T), rows, np.arange(k.shape[0]), off)
    L = _lse(s)
    return _probs(s, L) @ v, L[:, 0]


def head_backward_rows(q, k, v, do, scale, causal, q_rows, k_rows, row_block=ROW_BLOCK):
    """Gradients for sampled rows: dq at absolute query rows ``q_rows`` and
    dk, dv at absolute key rows ``k_rows``.

    The softmax term sum_k P_ik dP_ik needs whole rows, so it and LSE are
    formed for every query row (row_block rows at a time); the sampled
    gradients then follow the same definitions as ``head_backward``.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Sq = q.shape[0]
    off = causal_offset(causal, Sq, k.shape[0])
    lse = np.empty(Sq)
    psum = np.empty(Sq)
    for r0 in range(0, Sq, row_block):
        r1 = min(Sq, r0 + row_block)
        s = _scores(q[r0:r1], k, scale, off, r0)
        L = _lse(s)
        p = _probs(s, L)
        psum[r0:r1] = (p * (do[r0:r1] @ v.T)).sum(axis=1)
        lse[r0:r1] = L[:, 0]
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    # dq rows: full key range for each sampled query.
    s = _mask(scale * (q[q_rows] @ k.T), q_rows, np.arange(k.shape[0]), off)
    p = _probs(s, lse[q_rows][:, None])
    ds = p * (do[q_rows] @ v.T - psum[q_rows][:, None])
    dq = scale * (ds @ k)
    # dk, dv rows: full query range for each sampled key (columns of P).
    s = _mask(scale * (q @ k[k_rows].T), np.arange(Sq), k_rows, off)
    p = _probs(s, lse[:, None])
    dv = p.T @ do
    ds = p * (do @ v[k_rows].T - psum[:, None])
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def head_backward_qrows(q, k, v, do, scale, causal, rows):
    """dq at the given absolute query rows only.

    A query row's gradient needs nothing beyond its own full score row: its
    LSE, its probabilities and its softmax term sum_k P_ik dP_ik all come from
    that row, so this is the definition of ``head_backward`` restricted to the
    sampled rows (the key-side gradients, which need every row, are what
    ``head_backward_rows`` is for).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    rows = np.asarray(rows, dtype=np.int64)
    off = causal_offset(causal, q.shape[0], k.shape[0])
    s = _mask(scale * (q[rows] @ k.T), rows, np.arange(k.shape[0]), off)
    p = _probs(s, _lse(s))
    dp = do[rows] @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return scale * (ds @ k)
