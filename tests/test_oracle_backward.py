"""Pins for the gradient oracle (oracle.backward), each fixed by something
other than the oracle itself:

* central finite differences of the forward oracle (itself pinned against a
  50-digit brute force), for every input element of tiny problems, and for
  the scale;
* invariants the softmax fixes: the gradient w.r.t. the keys sums to zero
  (adding one vector to every key shifts a row's scores by a constant),
  the gradient w.r.t. the values sums to the sum of dO (rows of P sum to 1),
  sum_i q_i . dQ_i = sum_j k_j . dK_j (both equal sum_ij dS_ij S_ij);
* closed forms: constant V or a single key gives dQ = dK = 0, n = 1 gives
  dV = dO;
* an independent library routine (torch autograd of its own softmax);
* the samplers for full sizes against the full materialisation;
* planted mistakes that these pins must catch.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bwd_mod


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def one_head(x):
    return x[None, None]


def loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention(one_head(q), one_head(k), one_head(v), scale, causal)
    return float((o[0, 0] * do).sum())


def finite_difference(q, k, v, do, scale, causal, h=1e-6):
    grads = []
    for which in range(3):
        x = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(x[which])
        for idx in np.ndindex(g.shape):
            xp = [a.copy() for a in x]
            xm = [a.copy() for a in x]
            xp[which][idx] += h
            xm[which][idx] -= h
            g[idx] = (loss(*xp, do, scale, causal) - loss(*xm, do, scale, causal)) / (2 * h)
        grads.append(g)
    return grads


def grads(q, k, v, do, scale, causal):
    dq, dk, dv = oracle.attention_backward(one_head(q), one_head(k), one_head(v), one_head(do),
                                           scale, causal)
    return dq[0, 0], dk[0, 0], dv[0, 0]


def _fd_disagrees(cases=((5, 3, False), (5, 3, True))):
    for n, d, causal in cases:
        q, k, v, do = rnd((n, d), 1 + n), rnd((n, d), 2 + n), rnd((n, d), 3 + n), rnd((n, d), 4 + n)
        fd = finite_difference(q, k, v, do, 0.8, causal)
        an = grads(q, k, v, do, 0.8, causal)
        for a, b in zip(an, fd):
            if not np.allclose(a, b, rtol=1e-6, atol=1e-7):
                return True
    return False


@pytest.mark.parametrize("n,d,causal,scale", [(1, 4, False, 0.5), (2, 3, True, 1.0), (5, 4, False, 0.8),
                                              (6, 3, True, 0.8), (7, 2, True, 2.5)])
def test_matches_finite_differences(n, d, causal, scale):
    q, k, v, do = rnd((n, d), 10 + n), rnd((n, d), 20 + n), rnd((n, d), 30 + n), rnd((n, d), 40 + n)
    fd = finite_difference(q, k, v, do, scale, causal)
    for name, a, b in zip(("dQ", "dK", "dV"), grads(q, k, v, do, scale, causal), fd):
        assert np.allclose(a, b, rtol=1e-6, atol=1e-7), (name, np.abs(a - b).max())


@pytest.mark.parametrize("causal", [False, True])
def test_scale_derivative(causal):
    # dL/dscale = sum_ij dS_ij (q_i . k_j) = sum_i q_i . dQ_i / scale
    n, d, scale, h = 6, 4, 0.7, 1e-6
    q, k, v, do = rnd((n, d), 5), rnd((n, d), 6), rnd((n, d), 7), rnd((n, d), 8)
    fd = (loss(q, k, v, do, scale + h, causal) - loss(q, k, v, do, scale - h, causal)) / (2 * h)
    dq, _, _ = grads(q, k, v, do, scale, causal)
    assert abs((q * dq).sum() / scale - fd) <= 1e-7


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    n, d, scale = 60, 8, 0.35
    q, k, v, do = rnd((n, d), 11), rnd((n, d), 12), rnd((n, d), 13), rnd((n, d), 14)
    dq, dk, dv = grads(q, k, v, do, scale, causal)
    assert np.abs(dk.sum(axis=0)).max() <= 1e-12
    assert np.abs(dv.sum(axis=0) - do.sum(axis=0)).max() <= 1e-12
    assert abs((q * dq).sum() - (k * dk).sum()) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_closed_forms(causal):
    n, d = 9, 4
    q, k, do = rnd((n, d), 21), rnd((n, d), 22), rnd((n, d), 23)
    v = np.tile(rnd((1, d), 24), (n, 1))           # O does not depend on P
    dq, dk, dv = grads(q, k, v, do, 0.5, causal)
    assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
    one = [rnd((1, d), 30 + i) for i in range(4)]  # a single key: P = 1
    dq, dk, dv = grads(*one, 0.5, causal)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0 and np.allclose(dv, one[3], atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_agrees_with_torch_autograd(causal):
    b, h, n, d, scale = 2, 2, 70, 16, 0.3
    q, k, v, do = (rnd((b, h, n, d), 40 + i) for i in range(4))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = scale * tq @ tk.transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.tensor(do))
    mine = oracle.attention_backward(q, k, v, do, scale, causal)
    for a, t in zip(mine, (tq, tk, tv)):
        assert np.abs(a - t.grad.numpy()).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_samplers_equal_full_materialisation(causal):
    n, d, scale = 300, 16, 0.25
    q, k, v, do = rnd((n, d), 51), rnd((n, d), 52), rnd((n, d), 53), rnd((n, d), 54)
    dq, dk, dv = grads(q, k, v, do, scale, causal)
    rows = [0, 1, 77, 150, 299]
    dq_r, _ = oracle.backward_rows(q, k, v, do, scale, causal, rows, block=64)
    assert np.abs(dq_r - dq[rows]).max() <= 1e-12
    lse, dsum = oracle.head_statistics(q, k, v, do, scale, causal, block=64)
    cols = [0, 5, 150, 298, 299]
    dk_c, dv_c = oracle.backward_key_columns(q, k, v, do, scale, causal, cols, lse, dsum)
    assert np.abs(dk_c - dk[cols]).max() <= 1e-12
    assert np.abs(dv_c - dv[cols]).max() <= 1e-12
    # D is also dO_i . O_i when O = P V exactly
    o, _ = oracle.attention(one_head(q), one_head(k), one_head(v), scale, causal)
    assert np.abs(dsum - (do * o[0, 0]).sum(axis=1)).max() <= 1e-12


# ---------------------------------------------------------------- planted mistakes

def test_pins_catch_planted_mistakes(monkeypatch):
    assert not _fd_disagrees()
    orig_sg = bwd_mod._softmax_grad
    orig_scg = bwd_mod._score_grads
    orig_p = bwd_mod._probabilities
    softmax_mutants = {
        "dropped -D term": lambda p, dp: (p * dp, (p * dp).sum(axis=1)),
        "D summed over the wrong axis": lambda p, dp: (p * (dp - (p * dp).sum(axis=0)[None, :]),
                                                       (p * dp).sum(axis=0)),
        "sign of D flipped": lambda p, dp: (p * (dp + (p * dp).sum(axis=1)[:, None]),
                                            (p * dp).sum(axis=1)),
    }
    for name, fn in softmax_mutants.items():
        monkeypatch.setattr(bwd_mod, "_softmax_grad", fn)
        assert _fd_disagrees(), name
        monkeypatch.setattr(bwd_mod, "_softmax_grad", orig_sg)
    score_mutants = {
        "dQ and dK swapped": lambda ds, q, k, s: (float(s) * (ds.T @ q), float(s) * (ds @ k)),
        "dS not transposed for dK": lambda ds, q, k, s: (float(s) * (ds @ k), float(s) * (ds @ q)),
        "scale dropped": lambda ds, q, k, s: (ds @ k, ds.T @ q),
    }
    for name, fn in score_mutants.items():
        monkeypatch.setattr(bwd_mod, "_score_grads", fn)
        assert _fd_disagrees(), name
        monkeypatch.setattr(bwd_mod, "_score_grads", orig_scg)

    def diag_excluded(q, k, scale, causal, rows):
        s = float(scale) * (q[rows] @ k.T)
        if causal:
            s = np.where(np.arange(k.shape[0])[None, :] >= rows[:, None], -1e30, s)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        return e / e.sum(axis=1, keepdims=True)
    monkeypatch.setattr(bwd_mod, "_probabilities", diag_excluded)
    assert _fd_disagrees(((5, 3, True),)), "causal mask off by one"
    monkeypatch.setattr(bwd_mod, "_probabilities", orig_p)
    assert not _fd_disagrees()
