"""Pins for the oracle's target computation (LSE pass and future mass).

Nothing here compares the oracle with itself: every expected value comes from
a hand-worked fixture (tests/golden/target_hand.json), the dense brute force
of oracle/brute.py (a different route: the full S x S matrix read with masks),
a closed form, or an identity the definitions imply.

KVpop summary sections: App. D.1 (dense target identity), D.2 (transposed
attention with the mask d >= t + w), D.4 (implementation steps), B.1 (group
aggregation), B.2 (count normalisation, finite lookahead).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import digamma, logsumexp

import oracle
from oracle import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(B, Hq, Hkv, S, D, seed, std=1.0):
    r = np.random.default_rng(seed)
    q = (r.standard_normal((B, Hq, S, D)) * std).astype(np.float32)
    k = (r.standard_normal((B, Hkv, S, D)) * std).astype(np.float32)
    return q, k


def harmonic(n):
    """H_n through the digamma function (H_n = psi(n+1) + Euler gamma)."""
    return digamma(np.asarray(n, np.float64) + 1.0) + np.euler_gamma


# ---------------------------------------------------------------- golden


def test_golden_hand_worked_target():
    g = json.load(open(os.path.join(GOLD, "target_hand.json")))
    q = np.array(g["q"], np.float32)
    k = np.array(g["k"], np.float32)
    ls = oracle.lse(q, k, scale=g["scale"])
    np.testing.assert_allclose(ls, np.array(g["lse"]), atol=1e-6)
    for w, exp in g["mass_head0"].items():
        m, ph = oracle.future_mass(q, k, ls, int(w), scale=g["scale"], per_head=True)
        np.testing.assert_allclose(ph[0, 0, :, 0], exp, atol=1e-6)
    m, ph = oracle.future_mass(q, k, ls, 0, scale=g["scale"], per_head=True)
    np.testing.assert_allclose(ph[0, 0, :, 1], g["mass_head1_w0"], atol=1e-6)
    for agg, exp in g["group_w0"].items():
        m = oracle.future_mass(q, k, ls, 0, agg=agg, scale=g["scale"])
        np.testing.assert_allclose(m[0, 0], exp, atol=1e-6)
    m = oracle.future_mass(q, k, ls, 0, agg="sum", count_normalize=True, scale=g["scale"])
    np.testing.assert_allclose(m[0, 0], g["group_w0_sum_count_normalized"], atol=1e-6)


# ---------------------------------------------------------------- brute force


@pytest.mark.parametrize("B,Hq,Hkv,S,D,seed", [(1, 2, 1, 64, 16, 0), (2, 4, 2, 97, 32, 1),
                                               (1, 8, 2, 130, 64, 2), (1, 3, 3, 50, 8, 3)])
def test_lse_matches_dense_brute_force(B, Hq, Hkv, S, D, seed):
    q, k = _rand(B, Hq, Hkv, S, D, seed)
    np.testing.assert_allclose(oracle.lse(q, k), brute.lse(q, k), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("w", [0, 1, 5, 16, 63, 64, 100])
@pytest.mark.parametrize("lookahead", [-1, 0, 7])
def test_mass_matches_dense_brute_force(w, lookahead):
    B, Hq, Hkv, S, D = 1, 4, 2, 64, 16
    q, k = _rand(B, Hq, Hkv, S, D, 10 + w)
    ls = oracle.lse(q, k)
    ref_h = brute.mass_per_head(q, k, w, lookahead)
    for agg in ("sum", "mean", "max"):
        got, ph = oracle.future_mass(q, k, ls, w, lookahead=lookahead, agg=agg, per_head=True)
        np.testing.assert_allclose(ph, np.moveaxis(ref_h.reshape(B, Hkv, 2, S), 2, -1),
                                   rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(got, brute.aggregate(ref_h, Hkv, agg), rtol=1e-11, atol=1e-14)
        gotn = oracle.future_mass(q, k, ls, w, lookahead=lookahead, agg=agg, count_normalize=True)
        n = brute.count(S, w, lookahead)
        refn = np.where(n > 0, brute.aggregate(ref_h, Hkv, agg) / np.maximum(n, 1), 0.0)
        np.testing.assert_allclose(gotn, refn, rtol=1e-11, atol=1e-14)


def test_sampled_rows_and_columns_equal_full_arrays():
    B, Hq, Hkv, S, D = 2, 4, 2, 80, 32
    q, k = _rand(B, Hq, Hkv, S, D, 5)
    full = oracle.lse(q, k)
    rows = np.array([0, 5, 79, 80, 200, B * Hq * S - 1])
    np.testing.assert_array_equal(oracle.lse(q, k, rows=rows), full.reshape(-1)[rows])
    m = oracle.future_mass(q, k, full, 7)
    cols = np.array([0, 3, 79, 80, 150, B * Hkv * S - 1])
    np.testing.assert_array_equal(oracle.future_mass(q, k, full, 7, cols=cols), m.reshape(-1)[cols])


# ---------------------------------------------------------------- closed forms


def test_zero_queries_closed_forms():
    """q = 0 makes every causal row uniform: LSE_d = ln(d+1) and
    m_t = sum_{d=t+w}^{S-1} 1/(d+1) = H_S - H_{t+w}."""
    B, Hq, Hkv, S, D, w = 1, 4, 2, 300, 64, 9
    _, k = _rand(B, Hq, Hkv, S, D, 7)
    q = np.zeros((B, Hq, S, D), np.float32)
    ls = oracle.lse(q, k)
    np.testing.assert_allclose(ls, np.broadcast_to(np.log(np.arange(1, S + 1)), ls.shape), rtol=1e-13)
    t = np.arange(S)
    exp_m = np.where(t + w < S, harmonic(S) - harmonic(np.minimum(t + w, S)), 0.0)
    m, ph = oracle.future_mass(q, k, ls, w, per_head=True)
    np.testing.assert_allclose(ph[0, 0, :, 0], exp_m, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(m[0, 1], 2 * exp_m, rtol=1e-11, atol=1e-14)
    n = np.clip(S - t - w, 0, None)
    mn = oracle.future_mass(q, k, ls, w, count_normalize=True)
    np.testing.assert_allclose(mn[0, 0], np.where(n > 0, 2 * exp_m / np.maximum(n, 1), 0),
                               rtol=1e-11, atol=1e-14)


def test_first_row_normalizer_is_its_own_score():
    q, k = _rand(2, 4, 2, 40, 32, 8)
    ls = oracle.lse(q, k)
    for b in range(2):
        for g in range(4):
            z00 = float(np.dot(q[b, g, 0].astype(np.float64), k[b, g // 2, 0])) / math.sqrt(32)
            assert abs(ls[b, g, 0] - z00) < 1e-12


# ---------------------------------------------------------------- invariants


def test_rows_sum_to_one():
    q, k = _rand(1, 4, 2, 120, 64, 9)
    ls = oracle.lse(q, k)
    z = brute.scores(q, k)
    p = np.where(brute.causal_mask(120), np.exp(z - ls[..., None]), 0.0)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-12)


@pytest.mark.parametrize("S", [1, 2, 257, 700])
def test_zero_window_total_mass_equals_query_count(S):
    """With w = 0 and no lookahead every query's probabilities are all
    counted, so the mass of one head summed over keys is S; SUM over a group
    of G heads gives G*S."""
    q, k = _rand(1, 8, 2, S, 64, S)
    ls = oracle.lse(q, k)
    m, ph = oracle.future_mass(q, k, ls, 0, per_head=True)
    np.testing.assert_allclose(ph.sum(axis=2), S, rtol=1e-11)
    np.testing.assert_allclose(m.sum(axis=-1), 4 * S, rtol=1e-11)


@pytest.mark.parametrize("w", [1, 4, 33])
def test_windowed_total_mass_identity(w):
    """Sum_t m_t = sum_{d>=w} (1 - mass that row d puts on its own window)."""
    S = 150
    q, k = _rand(1, 2, 1, S, 32, 20 + w)
    ls = oracle.lse(q, k)
    _, ph = oracle.future_mass(q, k, ls, w, per_head=True)
    p = brute.probs(q, k)
    for g in range(2):
        expect = sum(1.0 - p[0, g, d, d - w + 1:d + 1].sum() for d in range(w, S))
        assert abs(ph[0, 0, :, g].sum() - expect) < 1e-10


def test_two_routes_log_mass():
    """App. D.2: log m_t is a log-sum-exp over future queries of z - LSE_d
    (the transposed-attention route); it equals the log of the column sum."""
    S, w = 90, 6
    q, k = _rand(1, 2, 1, S, 16, 31)
    ls = oracle.lse(q, k)
    _, ph = oracle.future_mass(q, k, ls, w, per_head=True)
    z = brute.scores(q, k)
    for g in range(2):
        for t in range(S - w):
            route = logsumexp(z[0, g, t + w:, t] - ls[0, g, t + w:])
            assert abs(route - math.log(ph[0, 0, t, g])) < 1e-10


def test_keys_inside_final_window_get_zero():
    S, w = 64, 10
    q, k = _rand(1, 4, 2, S, 16, 41)
    ls = oracle.lse(q, k)
    m = oracle.future_mass(q, k, ls, w)
    assert np.all(m[..., S - w:] == 0.0)
    assert np.all(m[..., :S - w] > 0.0)


def test_aggregation_relations():
    S, w = 100, 3
    q, k = _rand(1, 8, 2, S, 32, 51)
    ls = oracle.lse(q, k)
    s = oracle.future_mass(q, k, ls, w, agg="sum")
    mean = oracle.future_mass(q, k, ls, w, agg="mean")
    mx = oracle.future_mass(q, k, ls, w, agg="max")
    G = 4
    np.testing.assert_allclose(mean, s / G, rtol=1e-14)
    assert np.all(mx <= s + 1e-15) and np.all(s <= G * mx + 1e-12)
    # one head per group: all three modes agree
    q1, k1 = _rand(1, 2, 2, S, 32, 52)
    l1 = oracle.lse(q1, k1)
    a = [oracle.future_mass(q1, k1, l1, w, agg=x) for x in ("sum", "mean", "max")]
    np.testing.assert_array_equal(a[0], a[1])
    np.testing.assert_array_equal(a[0], a[2])


def test_lookahead_caps_count():
    S, w, L = 80, 4, 5
    q, k = _rand(1, 2, 1, S, 16, 61)
    ls = oracle.lse(q, k)
    mn = oracle.future_mass(q, k, ls, w, lookahead=L, count_normalize=True, agg="max")
    assert np.all(mn <= 1.0 + 1e-12)  # an average of probabilities
    m_inf = oracle.future_mass(q, k, ls, w, agg="max")
    m_l = oracle.future_mass(q, k, ls, w, lookahead=L, agg="max")
    assert np.all(m_l <= m_inf + 1e-15)
