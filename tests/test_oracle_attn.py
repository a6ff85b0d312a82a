"""Pins for the oracle's attention output of the main pass (dense causal
and over the running top-k mask).

KVpop summary (arXiv 2607.05061v2, paperlayer.ai): App. D.4, first step (the
model's main attention pass, whose normalizers the target reuses) and
App. I (the sparse student attention over the fixed-budget mask of
App. C.1).  O_d = sum over the retained keys t of R_d of
exp(z_dt - LSE_d) v_t, with z_dt = q_d . k_t / sqrt(D).

The oracle builds each row from a column loop; these tests pin it against
a dense float64 softmax-times-V brute force (the S x S matrix, masked),
closed forms (constant V, zero queries, the first row) and the invariants of
a convex combination, so a dropped diagonal, a wrong head map, a wrong
normalizer or a transposed V fails at least one of them.
"""
import numpy as np
import pytest

import oracle
from oracle import brute


def _inputs(B, Hq, Hkv, S, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    return q, k, v


def _members(sc, s, w, budget, lds, S):
    B, Hkv = sc.shape[:2]
    mem = np.zeros((B, Hkv, S, S), bool)
    for b in range(B):
        for h in range(Hkv):
            R, _ = brute.running_sets(sc[b, h], s, w, budget, float(lds[h]))
            for d in range(S):
                mem[b, h, d, sorted(R[d])] = True
    return mem


@pytest.mark.parametrize("B,Hq,Hkv,S,D", [(2, 4, 2, 37, 16), (1, 3, 1, 64, 8), (1, 8, 8, 20, 32)])
def test_dense_matches_brute_force(B, Hq, Hkv, S, D):
    q, k, v = _inputs(B, Hq, Hkv, S, D, seed=S + D)
    o, oa, ls = oracle.attn_out(q, k, v)
    causal = np.broadcast_to(brute.causal_mask(S), (B, Hkv, S, S))
    ro, rl = brute.attn_masked(q, k, v, causal)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ls, rl, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ls, oracle.lse(q, k), rtol=0, atol=1e-12)
    # the magnitude bound of a convex combination
    assert (oa >= np.abs(o) - 1e-12).all()
    oa_ref, _ = brute.attn_masked(q, k, np.abs(v), causal)
    np.testing.assert_allclose(oa, oa_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("S,s,w,budget,G", [(64, 4, 8, 24, 2), (48, 0, 4, 12, 1), (33, 2, 0, 9, 3)])
def test_sparse_matches_masked_brute_force(S, s, w, budget, G):
    B, Hkv, D = 2, 2, 16
    q, k, v = _inputs(B, Hkv * G, Hkv, S, D, seed=3 * S + budget)
    sc = np.random.default_rng(S).standard_normal((B, Hkv, S)).astype(np.float32)
    lds = np.array([0.0, 0.02], np.float32)
    o, _, ls = oracle.attn_out(q, k, v, sc, s, w, budget, log_decay=lds)
    ro, rl = brute.attn_masked(q, k, v, _members(sc, s, w, budget, lds, S))
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ls, rl, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ls, oracle.lse_sparse(q, k, sc, s, w, budget, log_decay=lds),
                               rtol=0, atol=1e-12)


def test_closed_forms():
    B, Hq, Hkv, S, D = 1, 4, 2, 50, 8
    q, k, v = _inputs(B, Hq, Hkv, S, D, seed=9)
    sc = np.random.default_rng(1).standard_normal((B, Hkv, S)).astype(np.float32)
    # constant V per channel: every convex combination returns it
    vc = np.broadcast_to(np.arange(D, dtype=np.float32) - 3.5, (B, Hkv, S, D)).copy()
    for args in ((), (sc, 2, 4, 16)):
        o, _, _ = oracle.attn_out(q, k, vc, *args)
        np.testing.assert_allclose(o, np.broadcast_to(np.arange(D) - 3.5, o.shape), rtol=0, atol=1e-12)
    # the first row attends only to itself
    o, _, _ = oracle.attn_out(q, k, v)
    G = Hq // Hkv
    for g in range(Hq):
        np.testing.assert_array_equal(o[0, g, 0], v[0, g // G, 0].astype(np.float64))
    # zero queries: uniform weights, the running mean of V
    o, _, ls = oracle.attn_out(np.zeros_like(q), k, v)
    cm = np.cumsum(v.astype(np.float64), axis=2) / np.arange(1, S + 1)[None, None, :, None]
    for g in range(Hq):
        np.testing.assert_allclose(o[0, g], cm[0, g // G], rtol=0, atol=1e-12)
    np.testing.assert_allclose(ls[0, 0], np.log(np.arange(1, S + 1)), rtol=0, atol=1e-12)


def test_sparse_without_eviction_is_dense_and_rows_sample():
    B, Hq, Hkv, S, D = 2, 4, 2, 40, 16
    q, k, v = _inputs(B, Hq, Hkv, S, D, seed=4)
    sc = np.random.default_rng(2).standard_normal((B, Hkv, S)).astype(np.float32)
    dense = oracle.attn_out(q, k, v)
    never = oracle.attn_out(q, k, v, sc, 4, 8, S + 12)  # the budget holds every token
    np.testing.assert_allclose(never[0], dense[0], rtol=0, atol=1e-12)
    rows = np.array([0, 7, S - 1, S + 5, B * Hq * S - 1], np.int64)
    for full, args in ((dense, ()), (oracle.attn_out(q, k, v, sc, 2, 4, 12), (sc, 2, 4, 12))):
        o, oa, ls = oracle.attn_out(q, k, v, *args, rows=rows)
        np.testing.assert_array_equal(o, full[0].reshape(-1, D)[rows])
        np.testing.assert_array_equal(oa, full[1].reshape(-1, D)[rows])
        np.testing.assert_array_equal(ls, full[2].reshape(-1)[rows])
