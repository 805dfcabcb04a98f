"""Pins for the CPU oracle: it is checked against things other than itself.

Each test names what fixes the expected value: a 50-digit brute force of the
definition, a closed form, an invariant of softmax, the online-softmax
identity, the associativity of the state merge, the figures printed on the
slides, or an independent library routine. Several tests plant a mistake in
the oracle (on the CPU) and check that the pins catch it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import reference as att_mod
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def one_head(x):
    return x[None, None]


# ---------------------------------------------------------------- formats

def test_decode_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])


def test_decode_e4m3fn_format_landmarks():
    # OCP E4M3 "fn": bias 7, subnormals m*2^-9, max 448, NaN only at S.1111.111
    table = {0x00: 0.0, 0x80: -0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
             0x38: 1.0, 0x3C: 1.5, 0x7E: 448.0, 0xFE: -448.0, 0x78: 256.0}
    for code, val in table.items():
        assert oracle.decode_e4m3fn(np.array([code], np.uint8))[0] == val
    assert np.isnan(oracle.decode_e4m3fn(np.array([0x7F, 0xFF], np.uint8))).all()


def test_decode_bf16_and_f16_match_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 16, size=4096, dtype=np.uint16)
    for fmt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        mine = oracle.decode(bits, fmt)
        ref = torch.from_numpy(bits.view(np.int16).copy()).view(tdt).to(torch.float64).numpy()
        ok = ~np.isnan(ref)
        assert np.array_equal(np.isnan(mine), np.isnan(ref))
        assert np.array_equal(mine[ok], ref[ok])
    # landmarks: bf16 0x3F80 = 1, 0xC000 = -2, 0x0001 = 2^-133
    assert list(oracle.decode_bf16(np.array([0x3F80, 0xC000, 0x0001], np.uint16))) == [1.0, -2.0, 2.0 ** -133]


def test_inputs_roundtrip_through_bits():
    inp = workload.make_inputs(1, 2, 5, 8, "fp8", seed=1, qk_mult=4.0)
    q = oracle.decode(inp.bits("q"), "fp8", inp.q_descale)
    ref = inp.q.to(torch.float64).numpy() * inp.q_descale
    assert np.array_equal(q, ref)
    # the encoding keeps the largest magnitude at the top code
    assert np.abs(oracle.decode(inp.bits("k"), "fp8")).max() == 448.0


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("n,d,causal,scale", [
    (1, 4, False, 0.5), (2, 3, True, 0.7), (5, 8, False, 1 / math.sqrt(8)),
    (7, 8, True, 1 / math.sqrt(8)), (16, 4, True, 0.37), (16, 6, False, 1.3),
])
def test_matches_decimal_brute_force(n, d, causal, scale):
    q, k, v = rnd((n, d), 10 + n), rnd((n, d), 20 + n), rnd((n, d + 1), 30 + n)
    o_ref, lse_ref = oracle.attention_decimal(q, k, v, scale, causal)
    o, lse = oracle.attention(one_head(q), one_head(k), one_head(v), scale, causal)
    np.testing.assert_allclose(o[0, 0], o_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], lse_ref, rtol=1e-13, atol=1e-13)


def test_matches_decimal_on_fp8_dequantised_inputs():
    inp = workload.make_inputs(1, 1, 12, 16, "fp8", seed=5, qk_mult=4.0)
    q = oracle.decode(inp.bits("q"), "fp8", inp.q_descale)[0, 0]
    k = oracle.decode(inp.bits("k"), "fp8", inp.k_descale)[0, 0]
    v = oracle.decode(inp.bits("v"), "fp8", inp.v_descale)[0, 0]
    for causal in (False, True):
        o_ref, lse_ref = oracle.attention_decimal(q, k, v, 0.25, causal)
        o, lse = oracle.attention(one_head(q), one_head(k), one_head(v), 0.25, causal)
        np.testing.assert_allclose(o[0, 0], o_ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[0, 0], lse_ref, rtol=1e-13, atol=1e-12)


def test_large_scores_do_not_overflow():
    # scores of order 1e4: exp would overflow without the max subtraction
    q, k, v = rnd((6, 4), 1, 100.0), rnd((6, 4), 2, 100.0), rnd((6, 4), 3)
    o_ref, lse_ref = oracle.attention_decimal(q, k, v, 1.0, True)
    o, lse = oracle.attention(one_head(q), one_head(k), one_head(v), 1.0, True)
    assert np.isfinite(o).all()
    np.testing.assert_allclose(o[0, 0], o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], lse_ref, rtol=1e-14)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    q, k, v = rnd((1, 2, 40, 16), 1), rnd((1, 2, 40, 16), 2), rnd((1, 2, 40, 16), 3)
    _, _, p = oracle.attention(q, k, v, 0.25, causal, return_p=True)
    assert np.abs(p.sum(-1) - 1).max() <= 1e-12
    assert (p >= 0).all()
    if causal:
        assert (np.triu(p[0, 0], 1) == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_that_row(causal):
    q, k = rnd((1, 1, 33, 8), 4), rnd((1, 1, 33, 8), 5)
    u = rnd((5,), 6)
    v = np.broadcast_to(u, (1, 1, 33, 5)).copy()
    o, _ = oracle.attention(q, k, v, 0.4, causal)
    assert np.abs(o - u).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_values(causal):
    n, d = 21, 8
    q, v = rnd((1, 1, n, d), 7), rnd((1, 1, n, 6), 8)
    kappa = rnd((d,), 9)
    k = np.broadcast_to(kappa, (1, 1, n, d)).copy()
    o, lse = oracle.attention(q, k, v, 0.3, causal)
    for i in range(n):
        vis = i + 1 if causal else n
        assert np.abs(o[0, 0, i] - v[0, 0, :vis].mean(0)).max() <= 1e-12
        s_i0 = 0.3 * float(q[0, 0, i] @ kappa)
        assert abs(lse[0, 0, i] - (s_i0 + math.log(vis))) <= 1e-12


def test_permuting_keys_with_values_changes_nothing():
    n = 50
    q, k, v = rnd((1, 1, n, 8), 11), rnd((1, 1, n, 8), 12), rnd((1, 1, n, 8), 13)
    perm = np.random.default_rng(14).permutation(n)
    o1, l1 = oracle.attention(q, k, v, 0.5, False)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    assert np.abs(o1 - o2).max() <= 1e-12 and np.abs(l1 - l2).max() <= 1e-12
    # with a mask, the mask's columns move together with the keys
    excl = np.triu(np.ones((n, n), bool), 1)
    mask = np.where(excl, -np.inf, 0.0)
    o3, l3 = oracle.attention(q, k, v, 0.5, False, mask=mask)
    o4, l4 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.5, False, mask=mask[:, perm])
    assert np.abs(o3 - o4).max() <= 1e-12 and np.abs(l3 - l4).max() <= 1e-12


def test_causal_equals_explicit_additive_mask():
    n = 37
    q, k, v = rnd((2, 2, n, 8), 15), rnd((2, 2, n, 8), 16), rnd((2, 2, n, 8), 17)
    mask = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, 0.0)
    o1, l1 = oracle.attention(q, k, v, 0.3, True)
    o2, l2 = oracle.attention(q, k, v, 0.3, False, mask=mask)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_lse_is_consistent_with_scores_and_output():
    n = 30
    q, k, v = rnd((1, 1, n, 8), 18), rnd((1, 1, n, 8), 19), rnd((1, 1, n, 8), 20)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, 0.6, causal)
        s = 0.6 * q[0, 0] @ k[0, 0].T
        if causal:
            s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
        w = np.exp(s - lse[0, 0][:, None])
        assert np.abs(w.sum(1) - 1).max() <= 1e-12
        assert np.abs(w @ v[0, 0] - o[0, 0]).max() <= 1e-12


def test_special_cases():
    q, k, v = rnd((1, 1, 1, 8), 21), rnd((1, 1, 1, 8), 22), rnd((1, 1, 1, 8), 23)
    o, lse = oracle.attention(q, k, v, 0.5, False)
    assert np.array_equal(o, v)
    assert lse[0, 0, 0] == pytest.approx(0.5 * float(q[0, 0, 0] @ k[0, 0, 0]), abs=1e-14)
    n = 19
    q, k, v = rnd((1, 1, n, 8), 24), rnd((1, 1, n, 8), 25), rnd((1, 1, n, 8), 26)
    o, lse = oracle.attention(q, k, v, 0.5, True)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])          # causal row 0 sees only key 0
    assert lse[0, 0, 0] == pytest.approx(0.5 * float(q[0, 0, 0] @ k[0, 0, 0]), abs=1e-14)
    # scale 0: uniform weights over the visible keys
    o, lse = oracle.attention(q, k, v, 0.0, True)
    prefix = np.cumsum(v[0, 0], 0) / np.arange(1, n + 1)[:, None]
    assert np.abs(o[0, 0] - prefix).max() <= 1e-13
    assert np.abs(lse[0, 0] - np.log(np.arange(1, n + 1))).max() <= 1e-13
    o, _ = oracle.attention(q, k, v, 0.0, False)
    assert np.abs(o[0, 0] - v[0, 0].mean(0)).max() <= 1e-13


def test_fully_excluded_row_reading():
    n = 4
    q, k, v = rnd((1, 1, n, 4), 27), rnd((1, 1, n, 4), 28), rnd((1, 1, n, 4), 29)
    mask = np.zeros((n, n))
    mask[2, :] = -np.inf
    o, lse = oracle.attention(q, k, v, 1.0, False, mask=mask)
    assert (o[0, 0, 2] == 0).all() and lse[0, 0, 2] == -np.inf
    assert np.isfinite(o[0, 0, [0, 1, 3]]).all()


def test_row_subset_and_block_size_do_not_change_rows():
    n = 70
    q, k, v = rnd((1, 2, n, 8), 30), rnd((1, 2, n, 8), 31), rnd((1, 2, n, 8), 32)
    o, lse = oracle.attention(q, k, v, 0.4, True)
    rows = [0, 5, 63, 64, 69]
    o2, lse2 = oracle.attention(q, k, v, 0.4, True, rows=rows, block=2)
    assert np.abs(o[:, :, rows] - o2).max() <= 1e-14
    assert np.abs(lse[:, :, rows] - lse2).max() <= 1e-14


# ---------------------------------------------------------------- online softmax

def test_rescale_identity():
    # e^(s - m_old) * e^(m_old - m_new) = e^(s - m_new)
    rng = np.random.default_rng(33)
    s, m_old, m_new = rng.normal(size=1000), rng.normal(size=1000), rng.normal(size=1000) + 3
    lhs = np.exp(s - m_old) * np.exp(m_old - m_new)
    np.testing.assert_allclose(lhs, np.exp(s - m_new), rtol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_two_tile_online_merge_equals_one_pass_at_every_cut(causal):
    n = 16
    q, k, v = rnd((n, 8), 34), rnd((n, 8), 35), rnd((n, 5), 36)
    o_ref, lse_ref = oracle.attention(one_head(q), one_head(k), one_head(v), 0.45, causal)
    for cut in range(1, n):
        o, lse = oracle.online_attention(q, k, v, 0.45, causal, [0, cut, n])
        assert np.abs(o - o_ref[0, 0]).max() <= 1e-12
        assert np.abs(lse - lse_ref[0, 0]).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_random_multi_tile_partitions(causal):
    rng = np.random.default_rng(37)
    n = 45
    q, k, v = rnd((n, 8), 38, 3.0), rnd((n, 8), 39, 3.0), rnd((n, 8), 40)
    o_ref, lse_ref = oracle.attention(one_head(q), one_head(k), one_head(v), 0.7, causal)
    for _ in range(20):
        inner = sorted(rng.choice(np.arange(1, n), size=rng.integers(1, 10), replace=False))
        o, lse = oracle.online_attention(q, k, v, 0.7, causal, [0, *inner, n])
        assert np.abs(o - o_ref[0, 0]).max() <= 1e-12
        assert np.abs(lse - lse_ref[0, 0]).max() <= 1e-12


def test_merge_is_associative_with_identity():
    rng = np.random.default_rng(41)
    R, d = 9, 4

    def state(seed):
        g = np.random.default_rng(seed)
        return (g.normal(size=R) * 5, g.uniform(0.5, 3, size=R), g.normal(size=(R, d)))
    a, b, c = state(1), state(2), state(3)
    left = oracle.merge_states(oracle.merge_states(a, b), c)
    right = oracle.merge_states(a, oracle.merge_states(b, c))
    for x, y in zip(left, right):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-13)
    e = oracle.empty_state(R, d)
    for x, y in zip(oracle.merge_states(a, e), a):
        np.testing.assert_allclose(x, y, rtol=0, atol=0)
    for x, y in zip(oracle.merge_states(e, a), a):
        np.testing.assert_allclose(x, y, rtol=0, atol=0)
    del rng


def test_tile_states_merged_in_any_bracketing_equal_one_pass():
    n = 24
    q, k, v = rnd((n, 8), 42), rnd((n, 8), 43), rnd((n, 8), 44)
    o_ref, lse_ref = oracle.attention(one_head(q), one_head(k), one_head(v), 0.5, True)
    rows = np.arange(n)[:, None]
    tiles = [(0, 5), (5, 11), (11, 17), (17, 24)]
    st = [oracle.tile_state(q, k[a:b], v[a:b], 0.5, excluded=np.arange(a, b)[None, :] > rows)
          for a, b in tiles]
    # causal rows may have every key of a tile excluded: m = -inf, l = 0 there
    m = oracle.merge_states
    for combo in (m(m(m(st[0], st[1]), st[2]), st[3]), m(st[0], m(st[1], m(st[2], st[3]))),
                  m(m(st[0], st[1]), m(st[2], st[3])), m(m(st[3], st[1]), m(st[2], st[0]))):
        o, lse = oracle.finalize_state(combo)
        assert np.abs(o - o_ref[0, 0]).max() <= 1e-12
        assert np.abs(lse - lse_ref[0, 0]).max() <= 1e-12


# ---------------------------------------------------------------- library routines

@pytest.mark.parametrize("causal", [False, True])
def test_agrees_with_independent_library_routines(causal):
    from scipy.special import logsumexp
    b, h, n, d = 2, 3, 300, 64
    q, k, v = rnd((b, h, n, d), 45), rnd((b, h, n, d), 46), rnd((b, h, n, d), 47)
    o, lse = oracle.attention(q, k, v, 1 / 8, causal, block=128)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=1 / 8)
    assert np.abs(o - ref.numpy()).max() <= 1e-12
    s = (1 / 8) * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
    assert np.abs(lse - logsumexp(s, axis=-1)).max() <= 1e-12


# ---------------------------------------------------------------- accounting

def test_accounting_matches_the_slides():
    g = json.load(open(os.path.join(GOLDEN, "real_size_accounting.json")))
    assert g["model_dim"] // g["heads"] == g["d_k"]
    f = oracle.flops(1, g["heads"], g["n"], g["d_k"], causal=False)
    assert abs(f - g["gemm_flops_per_layer_approx"]) / g["gemm_flops_per_layer_approx"] <= g["approx_rel_tol"]
    assert f == 4 * 32 * 8192 ** 2 * 128
    assert oracle.score_matrix_ratio(g["n"], g["d_k"]) == g["s_p_over_qkvo"]
    assert oracle.flops(1, 32, 8192, 128, causal=True) == f / 2


# element type of O for each input type (include/fa.h: e4m3 inputs give bf16 O)
OUT_OF = {"f32": "f32", "f16": "f16", "bf16": "bf16", "fp8": "bf16"}


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16", "fp8"])
@pytest.mark.parametrize("shape", [(1, 1, 256, 64), (2, 3, 100, 128), (1, 32, 8192, 128), (2, 32, 2048, 128)])
def test_min_hbm_bytes_is_the_size_of_the_tensors(shape, dtype):
    """min_hbm_bytes against an independent count: the bytes of the Q, K, V
    tensors the input generator makes, plus those of the O and fp32 LSE
    tensors a caller allocates for them (e4m3 in, bf16 out included)."""
    b, h, n, d = shape
    small = (b, h, min(n, 64), d)
    inp = workload.make_inputs(*small, dtype, seed=0)
    per_row_in = sum(t.numel() * t.element_size() for t in (inp.q, inp.k, inp.v)) // (b * h * small[2])
    o = torch.empty(small, dtype=workload.torch_dtype(OUT_OF[dtype]))
    lse = torch.empty(small[:3], dtype=torch.float32)
    per_row_out = (o.numel() * o.element_size() + lse.numel() * lse.element_size()) // (b * h * small[2])
    assert oracle.min_hbm_bytes(b, h, n, d, dtype, OUT_OF[dtype]) == b * h * n * (per_row_in + per_row_out)
    # without the LSE, Q + K + V + O alone
    assert oracle.min_hbm_bytes(b, h, n, d, dtype, OUT_OF[dtype], with_lse=False) == \
        b * h * n * (per_row_in + o.element_size() * d)


@pytest.mark.parametrize("n", [1, 2, 7, 33])
@pytest.mark.parametrize("causal", [False, True])
def test_exp_count_is_the_number_of_visible_entries_of_p(n, causal):
    """exp_count against the materialised P of the oracle: one exponential per
    entry the mask leaves visible (the others are exp(-inf) = 0, never
    evaluated)."""
    b, h, d = 2, 3, 16
    q, k, v = (rnd((b, h, n, d), 300 + i) for i in range(3))
    _, _, p = oracle.attention(q, k, v, 0.25, causal, return_p=True)
    s = 0.25 * np.einsum("bhid,bhjd->bhij", q, k)
    if causal:
        s = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, s)
    visible = int(np.isfinite(s).sum())
    assert (p[np.isfinite(s)] > 0).all() and (p[~np.isfinite(s)] == 0).all()
    assert oracle.exp_count(b, h, n, causal) == visible


# ---------------------------------------------------------------- planted mistakes

def _brute_force_disagrees():
    """True if the oracle now disagrees with the decimal brute force somewhere."""
    for n, d, causal in ((6, 4, False), (6, 4, True)):
        q, k, v = rnd((n, d), 50 + n), rnd((n, d), 60 + n), rnd((n, d), 70 + n)
        o_ref, lse_ref = oracle.attention_decimal(q, k, v, 0.8, causal)
        o, lse = oracle.attention(one_head(q), one_head(k), one_head(v), 0.8, causal)
        if not (np.allclose(o[0, 0], o_ref, rtol=1e-12, atol=1e-12)
                and np.allclose(lse[0, 0], lse_ref, rtol=1e-12, atol=1e-12)):
            return True
    return False


def test_pins_catch_planted_mistakes(monkeypatch):
    assert not _brute_force_disagrees()
    score_mutants = {
        "transposed operand (K Q^T)": lambda q, k, s: float(s) * (k @ q.T),
        "dropped scale": lambda q, k, s: q @ k.T,
        "scale applied twice": lambda q, k, s: float(s) ** 2 * (q @ k.T),
        "sign flipped": lambda q, k, s: -float(s) * (q @ k.T),
    }
    orig_scores = att_mod._scores
    for name, fn in score_mutants.items():
        monkeypatch.setattr(att_mod, "_scores", fn)
        assert _brute_force_disagrees(), name
        monkeypatch.setattr(att_mod, "_scores", orig_scores)
    mask_mutants = {
        "diagonal excluded": lambda r, n: np.arange(n)[None, :] >= r[:, None],
        "future visible, past excluded": lambda r, n: np.arange(n)[None, :] < r[:, None],
    }
    orig_mask = att_mod._causal_excluded
    for name, fn in mask_mutants.items():
        monkeypatch.setattr(att_mod, "_causal_excluded", fn)
        assert _brute_force_disagrees(), name
        monkeypatch.setattr(att_mod, "_causal_excluded", orig_mask)
    orig_soft = att_mod._rows_softmax_times_v

    def unnormalised(s, v):
        o, lse, p = orig_soft(s, v)
        return o * np.exp(lse - s.max(axis=1))[:, None], lse, p

    def log2_lse(s, v):
        o, lse, p = orig_soft(s, v)
        return o, lse / np.log(2.0), p
    for name, fn in (("missing division by l", unnormalised), ("base-2 LSE", log2_lse)):
        monkeypatch.setattr(att_mod, "_rows_softmax_times_v", fn)
        assert _brute_force_disagrees(), name
        monkeypatch.setattr(att_mod, "_rows_softmax_times_v", orig_soft)
    assert not _brute_force_disagrees()
