"""Gradients of exact attention in float64 (test infrastructure only).

The forward map is the one of ``reference.attention`` (slides "Case study:
FlashAttention", slide "Attention is where tokens meet"):
    S = scale * Q K^T + mask,   P = softmax_rows(S),   O = P V.
Given the gradient dO of a scalar loss with respect to O, the chain rule
through these three steps gives, per (batch, head):

    dV   = P^T dO                               (O = P V, differentiated in V)
    dP   = dO V^T                               (O = P V, differentiated in P)
    dS   = P * (dP - rowsum(P * dP))            (softmax Jacobian, row by row:
                                                 dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik))
    dQ   = scale * dS K                         (S = scale Q K^T)
    dK   = scale * dS^T Q

Masked entries have P_ij = 0, so they contribute nothing. The pages only
state that the backward pass recomputes the attention matrix on-chip in two
passes instead of storing it (article "Mastering FlashAttention: The
Algebraic Foundation", technical deep dive); what it computes is this
gradient, written out here with S, P, dP and dS materialised in full.

Two helpers serve full-size checks that sample outputs: ``backward_rows``
gives dQ (and the row statistic D = rowsum(P * dP)) for chosen query rows,
materialising their full rows; ``backward_key_columns`` gives dK and dV for
chosen keys from the columns of P, written as P_ij = exp(S_ij - LSE_i) with
the per-row log-sum-exp (the same P: exp(S_ij - m_i) / l_i with
LSE_i = m_i + ln l_i).
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from .reference import attention


def _probabilities(q: np.ndarray, k: np.ndarray, scale: float, causal: bool,
                   rows: np.ndarray) -> np.ndarray:
    """Full rows of P for query rows ``rows`` of one head ([R, n])."""
    s = float(scale) * (q[rows] @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], -np.inf, s)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def _softmax_grad(p: np.ndarray, dp: np.ndarray):
    """dS = P * (dP - D) with D = rowsum(P * dP); returns (dS, D)."""
    d = (p * dp).sum(axis=1)
    return p * (dp - d[:, None]), d


def _score_grads(ds: np.ndarray, q: np.ndarray, k: np.ndarray, scale: float):
    """(dQ, dK) from dS for S = scale * Q K^T."""
    return float(scale) * (ds @ k), float(scale) * (ds.T @ q)


def attention_backward(q, k, v, do, scale: float, causal: bool = False):
    """dQ, dK, dV for q, k, v, do of shape [batch, heads, n, d_k] (float64).

    Materialises S, P, dP and dS ([n, n] per head, about 3 GB at n = 8192);
    meant for n up to 8192.
    """
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    b, h, n, d = q.shape
    assert n <= 8192, "full materialisation; use the row / column helpers beyond this"
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    rows = np.arange(n)
    for bi in range(b):
        for hi in range(h):
            qq, kk, vv, dd = q[bi, hi], k[bi, hi], v[bi, hi], do[bi, hi]
            p = _probabilities(qq, kk, scale, causal, rows)
            dv[bi, hi] = p.T @ dd
            ds, _ = _softmax_grad(p, dd @ vv.T)
            dq[bi, hi], dk[bi, hi] = _score_grads(ds, qq, kk, scale)
    return dq, dk, dv


def backward_rows(q, k, v, do, scale: float, causal: bool, rows: Iterable[int], block: int = 512):
    """dQ [R, d] and D = rowsum(P * dP) [R] for query rows ``rows`` of one head.

    Each row is complete (its full row of P and dP), so row blocks only bound
    memory.
    """
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    rows = np.asarray(list(rows), dtype=np.int64)
    dq = np.zeros((rows.size, q.shape[1]))
    dsum = np.zeros(rows.size)
    for r0 in range(0, rows.size, block):
        r = rows[r0:r0 + block]
        p = _probabilities(q, k, scale, causal, r)
        ds, dd = _softmax_grad(p, do[r] @ v.T)
        dq[r0:r0 + block] = float(scale) * (ds @ k)
        dsum[r0:r0 + block] = dd
    return dq, dsum


def backward_key_columns(q, k, v, do, scale: float, causal: bool, cols: Iterable[int],
                         lse: np.ndarray, dsum: np.ndarray):
    """dK [C, d] and dV [C, d] for keys ``cols`` of one head.

    lse, dsum: the per-row log-sum-exp and D = rowsum(P * dP) of all n rows
    (from ``reference.attention`` and ``backward_rows``). Column j of P is
    exp(S_:j - LSE) (0 where masked).
    """
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    cols = np.asarray(list(cols), dtype=np.int64)
    n = q.shape[0]
    s = float(scale) * (q @ k[cols].T)                      # [n, C]
    if causal:
        s = np.where(cols[None, :] > np.arange(n)[:, None], -np.inf, s)
    p = np.exp(s - np.asarray(lse, np.float64)[:, None])
    dp = do @ v[cols].T
    ds = p * (dp - np.asarray(dsum, np.float64)[:, None])
    return float(scale) * (ds.T @ q), p.T @ do


def head_statistics(q, k, v, do, scale: float, causal: bool, block: int = 512):
    """(LSE [n], D [n]) of one head, every row complete."""
    _, lse = attention(np.asarray(q)[None, None], np.asarray(k)[None, None],
                       np.asarray(v)[None, None], scale, causal, block=block)
    _, dsum = backward_rows(q, k, v, do, scale, causal, range(np.asarray(q).shape[0]), block)
    return lse[0, 0], dsum
