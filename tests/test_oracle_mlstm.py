"""Pins for the oracle's delayed stateful mLSTM scorer.

KVpop summary (arXiv 2607.05061v2, paperlayer.ai): App. A (recurrent linear
attention: a running key-value summary C_t and normalizer, rank-one updates),
App. E.1 (headwise input [k; v]), App. E.3 (mLSTM matrix memory and
normalizer with scalar input/forget gates from headwise projections, the
numerically stabilised form, Hedgehog features), App. E.4 (token u = q - w
is read out from the state through q; SiLU readout with a bias).

The oracle runs the stabilised recurrence; the pins are the unstabilised
recurrence written as explicit sums (a different route: no running max, the
floor max(|n.r|, 1)), closed forms for one token and for a zero output
layer, the stabiliser's scaling invariant, and the delay bookkeeping.
"""
import numpy as np
import pytest

import oracle
from oracle import brute


def _params(H, D, P, E, seed, bi=0.0, bf=2.0):
    rng = np.random.default_rng(seed)
    X = 2 * D
    p = {"wk": rng.standard_normal((H, P, X)) / np.sqrt(X),
         "wr": rng.standard_normal((H, P, X)) / np.sqrt(X),
         "wv": rng.standard_normal((H, E, X)) / np.sqrt(X),
         "wi": rng.standard_normal((H, X)) / np.sqrt(X),
         "bi": np.full(H, bi), "wf": rng.standard_normal((H, X)) / np.sqrt(X),
         "bf": np.full(H, bf), "wo": rng.standard_normal((H, E)) / np.sqrt(E),
         "bo": rng.standard_normal(H) * 0.1}
    return {a: np.asarray(b, np.float32) for a, b in p.items()}


def _kv(B, H, n, D, seed):
    rng = np.random.default_rng(seed + 100)
    return (rng.standard_normal((B, H, n, D)).astype(np.float32),
            rng.standard_normal((B, H, n, D)).astype(np.float32))


@pytest.mark.parametrize("bi,bf", [(0.0, 2.0), (20.0, -20.0), (-20.0, 20.0), (8.0, 0.0)])
@pytest.mark.parametrize("w", [0, 1, 7])
def test_matches_unstabilised_recurrence(bi, bf, w):
    B, H, n, D, P, E = 2, 2, 30, 8, 4, 6
    k, v = _kv(B, H, n, D, int(bi + bf + w))
    pr = _params(H, D, P, E, seed=w, bi=bi, bf=bf)
    got = oracle.mlstm_scores(k, v, pr, w)
    ref = brute.mlstm_scores_unstabilised(k, v, pr, w)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    # token u is scored exactly when u + w is a token of the sequence
    assert np.isnan(got[..., n - w:]).all() and not np.isnan(got[..., :n - w]).any()


def test_zero_output_layer_and_no_readout():
    k, v = _kv(1, 3, 20, 8, 1)
    pr = _params(3, 8, 4, 4, seed=2)
    pr["wo"][:] = 0
    sc = oracle.mlstm_scores(k, v, pr, 3)
    np.testing.assert_array_equal(sc[..., :17], np.broadcast_to(pr["bo"][None, :, None].astype(np.float64), (1, 3, 17)))
    assert np.isnan(oracle.mlstm_scores(k, v, _params(3, 8, 4, 4, seed=2), 20)).all()


def test_single_token_closed_form():
    """w = 0, one token: m = i, C = val phi^T, n = phi, so h = val (phi.r) /
    max(phi.r, exp(-i)); with phi.r >= exp(-i), h = val."""
    D, P, E = 8, 4, 5
    k, v = _kv(1, 1, 1, D, 3)
    pr = _params(1, D, P, E, seed=4, bi=30.0)
    x = np.concatenate([k[0, 0, 0], v[0, 0, 0]]).astype(np.float64)
    val = pr["wv"][0].astype(np.float64) @ x
    silu = val / (1 + np.exp(-val))
    want = pr["wo"][0].astype(np.float64) @ silu + float(pr["bo"][0])
    got = oracle.mlstm_scores(k, v, pr, 0)[0, 0, 0]
    assert abs(got - want) < 1e-12


def test_stabiliser_scales_state_by_exp_minus_m():
    """The final stabilised state equals the unstabilised sums times
    exp(-m_q), and each Hedgehog half of the key features sums to one, so
    sum_j n_j = 2 exp(-m) sum_t (decay_t exp(i_t))."""
    B, H, n, D, P, E = 1, 1, 12, 8, 4, 3
    k, v = _kv(B, H, n, D, 5)
    pr = _params(H, D, P, E, seed=6, bi=5.0, bf=1.0)
    _, (C, nr, m) = oracle.mlstm_scores(k, v, pr, 2, want_state=True)
    x = np.concatenate([k[0, 0], v[0, 0]], axis=-1).astype(np.float64)
    ig = x @ pr["wi"][0].astype(np.float64) + float(pr["bi"][0])
    fg = x @ pr["wf"][0].astype(np.float64) + float(pr["bf"][0])
    sf = 1 / (1 + np.exp(-fg))
    wgt = np.array([np.prod(sf[t + 1:]) for t in range(n)]) * np.exp(ig)
    np.testing.assert_allclose(nr[0, 0].sum(), 2 * wgt.sum() * np.exp(-m[0, 0]), rtol=1e-12)
    assert m[0, 0] >= ig[-1]
