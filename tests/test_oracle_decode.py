"""Pins for the oracle's decode-side pieces: attention over the retained
cache, the headwise MLP scorer and the bounded-cache decode step.

KVpop summary: Sec. 3 (attention over the retained set; scoring begins when
a token leaves the window), App. C.1 (decoding attends over retained cache
entries; B = s + w + k), App. E.2 (stateless headwise MLP scorer), App. E.4
(at query q the newly eligible token is u = q - w).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.stats import norm

import oracle
from oracle import brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_bits(x):
    """Round float32 to bf16 (nearest-even) and return the raw bits."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _state(B, Hkv, budget, D):
    return {"kc": np.zeros((B, Hkv, budget, D), np.uint16), "vc": np.zeros((B, Hkv, budget, D), np.uint16),
            "slot_pos": np.full((B, Hkv, budget), -1, np.int32),
            "slot_score": np.full((B, Hkv, budget), -np.inf, np.float32)}


# ---------------------------------------------------------------- decode attention


def test_decode_matches_brute_force():
    r = np.random.default_rng(0)
    B, Hq, Hkv, n, D = 2, 8, 2, 40, 32
    q = r.standard_normal((B, Hq, D)).astype(np.float32)
    kc = r.standard_normal((B, Hkv, n, D)).astype(np.float32)
    vc = r.standard_normal((B, Hkv, n, D)).astype(np.float32)
    sp = np.where(r.random((B, Hkv, n)) < 0.3, -1, np.arange(n)).astype(np.int32)
    o, ls = oracle.decode_attend(q, kc, vc, sp)
    o2, ls2 = brute.decode(q, kc, vc, sp)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ls, ls2, rtol=1e-12)


def test_decode_without_eviction_equals_dense_last_row():
    """Budget >= sequence length keeps every token, so attention over the
    cache is the dense causal attention of the last query."""
    r = np.random.default_rng(1)
    B, Hq, Hkv, S, D = 1, 4, 2, 70, 16
    s, w = 4, 8
    budget = 100
    q = r.standard_normal((B, Hq, S, D)).astype(np.float32)
    k = r.standard_normal((B, Hkv, S, D)).astype(np.float32)
    v = r.standard_normal((B, Hkv, S, D)).astype(np.float32)
    sp, _ = oracle.select(r.standard_normal((B, Hkv, S)).astype(np.float32), s, w, budget)
    assert ((sp >= 0).sum(-1) == S).all()
    o, ls = oracle.decode_attend(q[:, :, -1], oracle.gather(k, sp), oracle.gather(v, sp), sp)
    full = oracle.lse(q, k)
    np.testing.assert_allclose(ls, full[:, :, -1], rtol=1e-12)
    p = brute.probs(q, k)[:, :, -1]  # [B,Hq,S]
    o_ref = np.einsum("bgs,bgsd->bgd", p, brute.repeat_kv(v, 2))
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)


def test_decode_slot_permutation_invariance_and_empty():
    r = np.random.default_rng(2)
    B, Hq, Hkv, n, D = 1, 4, 1, 30, 16
    q = r.standard_normal((B, Hq, D)).astype(np.float32)
    kc = r.standard_normal((B, Hkv, n, D)).astype(np.float32)
    vc = r.standard_normal((B, Hkv, n, D)).astype(np.float32)
    sp = np.arange(n, dtype=np.int32)[None, None].copy()
    perm = r.permutation(n)
    o1, l1 = oracle.decode_attend(q, kc, vc, sp)
    o2, l2 = oracle.decode_attend(q, kc[:, :, perm], vc[:, :, perm], sp[:, :, perm])
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)
    o3, l3 = oracle.decode_attend(q, kc, vc, np.full_like(sp, -1))
    assert not o3.any() and np.all(l3 == -np.inf)


# ---------------------------------------------------------------- MLP scorer


def test_mlp_special_cases():
    r = np.random.default_rng(3)
    B, Hkv, n, D, hid = 2, 3, 10, 16, 8
    keys = r.standard_normal((B, Hkv, n, D)).astype(np.float32)
    z = np.zeros
    b2 = np.array([0.5, -1.0, 2.0], np.float32)
    # zero first layer: GELU(0) = 0, score = b2
    out = oracle.mlp_score(keys, z((Hkv, hid, D)), z((Hkv, hid)), r.standard_normal((Hkv, hid)), b2)
    np.testing.assert_allclose(out, np.broadcast_to(b2[None, :, None], out.shape), rtol=0, atol=0)
    # one unit reading coordinate c: score = k_c * Phi(k_c) (normal CDF route)
    for c in (0, 5):
        w1 = z((Hkv, hid, D), np.float32)
        w1[:, 0, c] = 1.0
        w2 = z((Hkv, hid), np.float32)
        w2[:, 0] = 1.0
        out = oracle.mlp_score(keys, w1, z((Hkv, hid)), w2, z(Hkv))
        x = keys[..., c].astype(np.float64)
        np.testing.assert_allclose(out, x * norm.cdf(x), rtol=1e-13, atol=1e-15)
    # linearity in the output layer
    w1 = r.standard_normal((Hkv, hid, D)).astype(np.float32)
    b1 = r.standard_normal((Hkv, hid)).astype(np.float32)
    wa = r.standard_normal((Hkv, hid)).astype(np.float32)
    wb = r.standard_normal((Hkv, hid)).astype(np.float32)
    sa = oracle.mlp_score(keys, w1, b1, wa, z(Hkv))
    sb = oracle.mlp_score(keys, w1, b1, wb, z(Hkv))
    sab = oracle.mlp_score(keys, w1, b1, wa.astype(np.float64) + wb, z(Hkv))
    np.testing.assert_allclose(sab, sa + sb, rtol=1e-6, atol=1e-6)


def test_gelu_known_value():
    """GELU(1) = Phi(1) = 0.8413447460685429 (standard normal table)."""
    keys = np.ones((1, 1, 1, 1), np.float32)
    out = oracle.mlp_score(keys, np.ones((1, 1, 1)), np.zeros((1, 1)), np.ones((1, 1)), np.zeros(1))
    assert abs(out[0, 0, 0] - 0.8413447460685429) < 1e-15


# ---------------------------------------------------------------- cache step


def _nan_eq(a, b):
    a = np.asarray(a, np.float32)
    b = np.array([float("nan") if x == "nan" else x for x in b], np.float32)
    return np.array_equal(a, b, equal_nan=True)


def test_cache_step_golden():
    g = json.load(open(os.path.join(GOLD, "cache_step_hand.json")))
    s, w, budget, delay, D = 1, 2, 5, 1, 4
    pre = g["prefix"]
    sc = np.array(pre["scores"], np.float32)[None, None]
    sp, ss = oracle.select(sc, s, w, budget)
    assert sp[0, 0].tolist() == pre["slot_pos"]
    assert ss[0, 0].tolist() == pre["slot_score"]
    st = _state(1, 1, budget, D)
    st["slot_pos"][:] = sp
    st["slot_score"][:] = ss
    kbits = np.arange(100, dtype=np.uint16)
    for step in g["steps"]:
        q = step["q"]
        knew = np.full((1, 1, D), kbits[q], np.uint16)
        oracle.cache_step(st, knew, knew + 1, np.array([[step["score_r"]]], np.float32), s, w, delay, q)
        assert st["slot_pos"][0, 0].tolist() == step["slot_pos"], step["why"]
        assert _nan_eq(st["slot_score"][0, 0], step["slot_score"]), step["why"]
        # every valid non-sink slot carries the K/V of the token it names
        for j, p in enumerate(st["slot_pos"][0, 0]):
            if p >= 5:
                assert (st["kc"][0, 0, j] == kbits[p]).all() and (st["vc"][0, 0, j] == kbits[p] + 1).all()


@pytest.mark.parametrize("s,w,k,delay,kind", [(4, 16, 20, 5, "normal"), (1, 8, 6, 0, "ties"),
                                              (0, 4, 3, 3, "normal"), (2, 5, 0, 2, "normal"),
                                              (3, 12, 9, 11, "ties")])
def test_cache_step_replay_matches_recomputed_topk(s, w, k, delay, kind):
    """Evict-min with strict improvement is the incremental form of the
    static top-k: after every step the long-range pool must equal the top-k
    (score desc, position asc) of all tokens that have left the window."""
    r = np.random.default_rng(s * 100 + w)
    B, Hkv, D = 2, 2, 4
    budget = s + w + k
    S0, steps = 3 * budget, 80
    n_tot = S0 + steps
    if kind == "ties":
        sig = (r.integers(0, 4, size=(B, Hkv, n_tot)) * 0.5).astype(np.float32)
    else:
        sig = r.standard_normal((B, Hkv, n_tot)).astype(np.float32)
    kall = _bf16_bits(r.standard_normal((B, Hkv, n_tot, D)).astype(np.float32))
    vall = _bf16_bits(r.standard_normal((B, Hkv, n_tot, D)).astype(np.float32))
    sp, ss = oracle.select(sig[..., :S0], s, w, budget)
    st = {"kc": oracle.gather(kall[:, :, :S0], sp), "vc": oracle.gather(vall[:, :, :S0], sp),
          "slot_pos": sp, "slot_score": ss}
    for q in range(S0, n_tot):
        oracle.cache_step(st, kall[:, :, q], vall[:, :, q], sig[..., q - delay], s, w, delay, q)
        for b in range(B):
            for h in range(Hkv):
                row = st["slot_pos"][b, h]
                assert (row >= 0).sum() <= budget
                assert row[:s].tolist() == list(range(s))
                ring = sorted(int(p) for p in row[s + k:] if p >= 0)
                assert ring == list(range(q - w + 1, q + 1))
                exited = list(range(s, q - w + 1))
                order = sorted(exited, key=lambda t: (-float(sig[b, h, t]), t))[:k]
                assert sorted(int(p) for p in row[s:s + k] if p >= 0) == sorted(order)
                for j, p in enumerate(row):
                    if p >= 0:
                        assert st["kc"][b, h, j].tobytes() == kall[b, h, p].tobytes()
                        assert st["vc"][b, h, j].tobytes() == vall[b, h, p].tobytes()
                        if j >= s and p <= q - delay:
                            assert st["slot_score"][b, h, j] == sig[b, h, p]
