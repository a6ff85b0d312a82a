"""Pins for the oracle's running top-k mask and sparse log-normalizer.

KVpop summary (arXiv 2607.05061v2, paperlayer.ai): App. C.1 (the fixed-budget
mask keeps sinks, the protected window and the top-k of the eligible pool at
every query), App. C.2 (running cutoffs by a Fenwick tree), Sec. 3 and
App. B.3 (per-head decay as static priorities), App. D.3 (the target may
reuse the sparse attention's normalizer), App. F (fp32 ranking).

The oracle computes cutoffs with a Fenwick tree and derives keep_until from
them; these tests pin it against hand-worked rows, a per-query textbook sort
(Python's ``sorted``, a different route), closed forms for constant and
ramped scores, the one-shot retention at the last query, and, for the sparse
normalizer, dense masked brute force and the dense normalizer when nothing is
evicted.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_hand_worked_rows():
    g = json.load(open(os.path.join(GOLD, "running_topk_hand.json")))
    for c in g["cases"]:
        sc = np.array([[c["scores"]]], np.float32)
        ld = np.array([c["log_decay"]], np.float32)
        until, cut = oracle.running_topk(sc, c["s"], c["w"], c["budget"], log_decay=ld)
        assert until[0, 0].tolist() == c["keep_until"], c["name"]
        assert cut[0, 0].tolist() == c["cutoff"], c["name"]


KINDS = ["normal", "ties", "special", "const", "ramp", "nan"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("S,s,w,budget,lam", [(96, 4, 16, 40, 0.0), (80, 0, 0, 10, 0.0),
                                              (64, 2, 5, 20, 0.03), (50, 4, 16, 64, 0.0),
                                              (70, 1, 7, 9, 0.5), (40, 3, 0, 8, 0.0),
                                              (45, 2, 3, 5, 0.0)])
def test_running_topk_matches_per_query_sort(kind, S, s, w, budget, lam):
    sc = synth.scores((1, 2, S), seed=S * 7 + budget, kind=kind).numpy()
    ld = np.array([lam, 2 * lam], np.float32)
    until, cut = oracle.running_topk(sc, s, w, budget, log_decay=ld)
    for h in range(2):
        R, bcut = brute.running_sets(sc[0, h], s, w, budget, float(ld[h]))
        assert until[0, h].tolist() == brute.keep_until_from_sets(R, S)
        assert cut[0, h].tolist() == bcut
        for d in range(S):  # the mask's own invariants
            assert len(R[d]) <= budget
            assert set(range(min(s, d + 1))) <= R[d]
            assert set(range(max(d - w + 1, 0), d + 1)) <= R[d]


@pytest.mark.parametrize("kind", KINDS)
def test_last_query_equals_one_shot_retention(kind):
    """At the last query the pool is [s, S - w), the eligible set of the
    one-shot retention: both must keep the same tokens (no decay)."""
    S, s, w, budget = 300, 4, 32, 100
    sc = synth.scores((2, 3, S), seed=11, kind=kind).numpy()
    until, _ = oracle.running_topk(sc, s, w, budget)
    sp, _ = oracle.select(sc, s, w, budget)
    for b in range(2):
        for h in range(3):
            kept = sorted(t for t in range(S) if until[b, h, t] == S)
            assert kept == sorted(int(p) for p in sp[b, h] if p >= 0)


def test_closed_forms_constant_and_recency():
    S, s, w, budget = 200, 4, 16, 50
    k = budget - s - w
    # constant scores, no decay: ties keep the oldest k forever
    until, cut = oracle.running_topk(np.zeros((1, 1, S), np.float32), s, w, budget)
    exp_until = [S if t < s + k else min(t + w, S) for t in range(S)]
    assert until[0, 0].tolist() == exp_until
    first_full = s + k - 1 + w
    assert cut[0, 0].tolist() == [-1] * first_full + [s + k - 1] * (S - first_full)
    # constant scores with decay (and rising scores without): the newest k
    # of the pool are kept, so token t leaves when k newer tokens entered
    for sc, ld in ((np.zeros((1, 1, S), np.float32), np.array([0.1], np.float32)),
                   (np.arange(S, dtype=np.float32)[None, None], None)):
        until, cut = oracle.running_topk(sc, s, w, budget, log_decay=ld)
        assert until[0, 0].tolist() == [S if t < s else min(t + w + k, S) for t in range(S)]
        assert cut[0, 0].tolist() == [-1] * first_full + [d - w - k + 1 for d in range(first_full, S)]


def test_budget_zero_long_range_and_no_window():
    S = 40
    sc = synth.scores((1, 1, S), seed=3).numpy()
    until, cut = oracle.running_topk(sc, 2, 8, 10)  # k = 0: sinks + window only
    assert until[0, 0].tolist() == [S, S] + [min(t + 8, S) for t in range(2, S)]
    assert (cut == -1).all()
    until, cut = oracle.running_topk(sc, 0, 0, 5)  # w = 0: a token enters the pool at once
    R, bcut = brute.running_sets(sc[0, 0], 0, 0, 5)
    assert until[0, 0].tolist() == brute.keep_until_from_sets(R, S)
    assert cut[0, 0].tolist() == bcut


def _members(sc, s, w, budget, lds, S):
    B, Hkv = sc.shape[:2]
    mem = np.zeros((B, Hkv, S, S), bool)
    for b in range(B):
        for h in range(Hkv):
            R, _ = brute.running_sets(sc[b, h], s, w, budget, float(lds[h]))
            for d in range(S):
                mem[b, h, d, sorted(R[d])] = True
    return mem


@pytest.mark.parametrize("S,s,w,budget,G", [(64, 4, 8, 24, 2), (48, 0, 4, 12, 1), (33, 2, 0, 9, 3)])
def test_sparse_lse_matches_masked_brute_force(S, s, w, budget, G):
    rng = np.random.default_rng(S + budget)
    B, Hkv, D = 2, 2, 16
    q = rng.standard_normal((B, Hkv * G, S, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    sc = rng.standard_normal((B, Hkv, S)).astype(np.float32)
    lds = np.array([0.0, 0.02], np.float32)
    got = oracle.lse_sparse(q, k, sc, s, w, budget, log_decay=lds)
    ref = brute.lse_masked(q, k, _members(sc, s, w, budget, lds, S))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # sampled rows give the same values as the full array
    rows = np.array([0, 5, S - 1, S + 3, B * Hkv * G * S - 1], np.int64)
    np.testing.assert_array_equal(oracle.lse_sparse(q, k, sc, s, w, budget, log_decay=lds, rows=rows),
                                  got.reshape(-1)[rows])


def test_sparse_lse_reduces_to_dense_and_bounds_it():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, S, D = 1, 4, 2, 96, 32
    q = rng.standard_normal((B, Hq, S, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    sc = rng.standard_normal((B, Hkv, S)).astype(np.float32)
    dense = oracle.lse(q, k)
    # a budget that never evicts: R_d = [0, d]
    np.testing.assert_allclose(oracle.lse_sparse(q, k, sc, 4, 8, S + 12), dense, rtol=0, atol=1e-12)
    # evicting keeps a subset, so the sparse normalizer never exceeds the dense one
    sp = oracle.lse_sparse(q, k, sc, 4, 8, 30)
    assert (sp <= dense + 1e-12).all()
    assert (sp < dense - 1e-6).any()
    # rows whose whole causal prefix fits the budget are unchanged
    np.testing.assert_allclose(sp[..., :30], dense[..., :30], rtol=0, atol=1e-12)
