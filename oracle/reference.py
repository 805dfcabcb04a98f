"""Exact scaled-dot-product attention forward in float64 (test infrastructure only).

What is computed (the equation of the slide "Attention is where tokens meet"
in "Case study: FlashAttention", written per row as on the slide "Problem:
softmax needs the whole row"):

    S = scale * Q K^T + mask          (mask: 0 where visible, -inf where excluded)
    m_i = max_j S_ij
    l_i = sum_j exp(S_ij - m_i)
    P_ij = exp(S_ij - m_i) / l_i
    O = P V
    LSE_i = m_i + ln l_i              (the log-sum-exp of row i, natural log)

The causal mask excludes key j from query i when j > i. ``scale`` is used as
given; callers pass the fp32-rounded value the kernel receives. Natural
``exp`` is used on purpose (the kernel works in base 2 with log2(e) folded
into its scale), so that folding is checked rather than shared.

Rows are processed in blocks of whole rows: each block materialises its full
rows of S and P, which is the definition applied row by row (O_i depends on
row i of S only); blocks merely bound memory.

Readings where the pages are silent: a row with every key excluded cannot
occur with the causal mask (key i is always visible to query i), but for a
general mask it yields O_i = 0 and LSE_i = -inf.
"""
from __future__ import annotations

from decimal import Decimal, localcontext
from typing import Iterable, Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# one-pass definition
# --------------------------------------------------------------------------

def _scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """scale * q k^T for q [R, d], k [n, d] -> [R, n] (float64)."""
    return float(scale) * (q @ k.T)


def _causal_excluded(rows: np.ndarray, n: int) -> np.ndarray:
    """True where key j is excluded for query rows[i], i.e. j > rows[i]."""
    return np.arange(n)[None, :] > rows[:, None]


def _rows_softmax_times_v(s: np.ndarray, v: np.ndarray):
    """Softmax over full rows of s (materialising P), then P v and the LSE."""
    m = s.max(axis=1)
    dead = ~np.isfinite(m)  # every key excluded (general masks only)
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    l = e.sum(axis=1)
    l_safe = np.where(dead, 1.0, l)
    p = e / l_safe[:, None]
    o = p @ v
    lse = np.where(dead, -np.inf, m_safe + np.log(l_safe))
    o[dead] = 0.0
    return o, lse, p


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
              mask: Optional[np.ndarray] = None, rows: Optional[Iterable[int]] = None,
              block: int = 512, return_p: bool = False):
    """O and LSE for q, k, v of shape [batch, heads, n, d_k] (float64).

    mask  -- optional additive mask broadcastable to [batch, heads, n, n].
    rows  -- optional query rows to evaluate (all rows if None); the causal
             mask uses each row's absolute index.
    Returns (O [b, h, R, d_k], LSE [b, h, R]) and, if ``return_p``, also
    P [b, h, R, n].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, h, n, d = q.shape
    assert k.shape == (b, h, n, d) and v.shape[:3] == (b, h, n)
    row_idx = np.arange(n) if rows is None else np.asarray(list(rows), dtype=np.int64)
    R = row_idx.size
    out = np.zeros((b, h, R, v.shape[3]), dtype=np.float64)
    lse = np.zeros((b, h, R), dtype=np.float64)
    pmat = np.zeros((b, h, R, n), dtype=np.float64) if return_p else None
    if mask is not None:
        mask = np.broadcast_to(np.asarray(mask, dtype=np.float64), (b, h, n, n))
    for bi in range(b):
        for hi in range(h):
            kk, vv = k[bi, hi], v[bi, hi]
            for r0 in range(0, R, block):
                ridx = row_idx[r0:r0 + block]
                s = _scores(q[bi, hi, ridx], kk, scale)
                if causal:
                    s[_causal_excluded(ridx, n)] = -np.inf
                if mask is not None:
                    s = s + mask[bi, hi][ridx]
                o, l, p = _rows_softmax_times_v(s, vv)
                out[bi, hi, r0:r0 + block] = o
                lse[bi, hi, r0:r0 + block] = l
                if return_p:
                    pmat[bi, hi, r0:r0 + block] = p
    if return_p:
        return out, lse, pmat
    return out, lse


# --------------------------------------------------------------------------
# online softmax: streaming over key tiles, and the associative merge
# --------------------------------------------------------------------------
# State per query row: (m, l, o) -- running max, running sum of exp(s - m)
# and the unnormalised output sum of exp(s - m) v. The empty state is
# (-inf, 0, 0).

def empty_state(rows: int, d_v: int):
    return (np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, d_v)))


def _exp_shift(a: np.ndarray, m: np.ndarray) -> np.ndarray:
    """exp(a - m) with exp(-inf - (-inf)) taken as 0 (nothing seen yet)."""
    with np.errstate(invalid="ignore"):
        r = np.exp(a - m)
    return np.where(np.isneginf(a), 0.0, r)


def online_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
                     cuts: Sequence[int], mask: Optional[np.ndarray] = None):
    """One head ([n, d] matrices), keys visited tile by tile.

    Tiles are [cuts[t], cuts[t+1]). Each tile applies the update of the slide
    "Online softmax: divide once, at the end":
        m_new = max(m, max over the tile of s)
        alpha = exp(m - m_new)
        l     = alpha * l + sum over the tile of exp(s - m_new)
        o     = alpha * o + sum over the tile of exp(s - m_new) v
    and after the last tile O = o / l (one division) and LSE = m + ln l.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n = q.shape[0]
    rows = np.arange(n)
    m, l, o = empty_state(n, v.shape[1])
    cuts = list(cuts)
    assert cuts[0] == 0 and cuts[-1] == k.shape[0] and all(a < b for a, b in zip(cuts, cuts[1:]))
    for a, b in zip(cuts, cuts[1:]):
        s = _scores(q, k[a:b], scale)
        if causal:
            s[np.arange(a, b)[None, :] > rows[:, None]] = -np.inf
        if mask is not None:
            s = s + np.asarray(mask, np.float64)[:, a:b]
        m_new = np.maximum(m, s.max(axis=1))
        alpha = _exp_shift(m, m_new)
        p = _exp_shift(s, m_new[:, None])
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + p @ v[a:b]
        m = m_new
    return finalize_state((m, l, o))


def tile_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
               excluded: Optional[np.ndarray] = None):
    """(m, l, o) of one key tile on its own, starting from the empty state."""
    s = _scores(np.asarray(q, np.float64), np.asarray(k, np.float64), scale)
    if excluded is not None:
        s = np.where(excluded, -np.inf, s)
    m = s.max(axis=1)
    p = _exp_shift(s, m[:, None])
    return (m, p.sum(axis=1), p @ np.asarray(v, np.float64))


def merge_states(a, b):
    """Combine two states over disjoint key sets.

    m = max(m_a, m_b); each side is rescaled by exp(m_side - m) before its
    l and o are added. This is the associative ("twisted monoid") operation
    that the article "Mastering FlashAttention: The Algebraic Foundation"
    identifies behind FlashAttention and safe softmax; (-inf, 0, 0) is its
    identity.
    """
    ma, la, oa = a
    mb, lb, ob = b
    m = np.maximum(ma, mb)
    ca = _exp_shift(ma, m)
    cb = _exp_shift(mb, m)
    return (m, ca * la + cb * lb, ca[:, None] * oa + cb[:, None] * ob)


def finalize_state(state):
    """O = o / l and LSE = m + ln l (rows with nothing visible: O = 0, LSE = -inf)."""
    m, l, o = state
    dead = l == 0
    l_safe = np.where(dead, 1.0, l)
    out = o / l_safe[:, None]
    out[dead] = 0.0
    lse = np.where(dead, -np.inf, m + np.log(l_safe))
    return out, lse


# --------------------------------------------------------------------------
# brute force in 50-digit decimal arithmetic (tiny inputs only)
# --------------------------------------------------------------------------

def attention_decimal(q, k, v, scale: float, causal: bool, prec: int = 50):
    """Element-by-element evaluation of the definition with ``decimal``.

    q, k, v: one head as nested sequences / arrays of floats ([n, d]); every
    float converts to Decimal exactly. Returns (O, LSE) as float64 arrays.
    Independent of NumPy's BLAS and exp.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    dv = v.shape[1]
    with localcontext() as ctx:
        ctx.prec = prec
        sc = Decimal(float(scale))
        Q = [[Decimal(float(x)) for x in row] for row in q]
        K = [[Decimal(float(x)) for x in row] for row in k]
        V = [[Decimal(float(x)) for x in row] for row in v]
        O = np.zeros((n, dv))
        LSE = np.zeros(n)
        for i in range(n):
            vis = [j for j in range(n) if not (causal and j > i)]
            s = {}
            for j in vis:
                acc = Decimal(0)
                for t in range(d):
                    acc += Q[i][t] * K[j][t]
                s[j] = sc * acc
            m = max(s.values())
            e = {j: (s[j] - m).exp() for j in vis}
            l = sum(e.values(), Decimal(0))
            for c in range(dv):
                acc = Decimal(0)
                for j in vis:
                    acc += (e[j] / l) * V[j][c]
                O[i, c] = float(acc)
            LSE[i] = float(m + l.ln())
    return O, LSE
