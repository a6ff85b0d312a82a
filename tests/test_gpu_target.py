"""GPU parity of the target computation (kvpop_fwd_lse, kvpop_future_attn_target)
against the CPU oracle, through the C ABI.

KVpop summary: App. D.1 (dense target identity), D.2 (transposed attention,
mask d >= t + w), D.4 (implementation steps), B.1 (group aggregation), B.2
(count normalisation, finite lookahead).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (LSE_ATOL, MASS_ATOL, MASS_RTOL, assert_close, ensure_built, f32,
                      group_problem, oracle_group_target)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    return ensure_built()


def _run(kv, q, k, window, **kw):
    lse = kv.fwd_lse(q, k)
    out = kv.future_attn_target(q, k, lse, window, per_qhead=True, **kw)
    torch.cuda.synchronize()
    return lse, out[0], out[1]


def _full_oracle(q, k, window, **kw):
    qf, kf = f32(q), f32(k)
    lse = oracle.lse(qf, kf)
    m, ph = oracle.future_mass(qf, kf, lse, window, per_head=True, **kw)
    return lse, m, ph


def _per_qhead(ph):  # oracle [B,Hkv,S,G] -> [B,Hq,S]
    B, Hkv, S, G = ph.shape
    return np.moveaxis(ph, 3, 2).reshape(B, Hkv * G, S)


def test_tiny_workload_full_parity(kv):
    w = synth.TINY
    q, k, _ = synth.attention_inputs(w, seed=1)
    q, k = q.cuda(), k.cuda()
    for window in (w.window, 0):
        lse, m, ph = _run(kv, q, k, window)
        olse, om, oph = _full_oracle(q, k, window)
        assert_close(f32(lse), olse, LSE_ATOL, 0, "lse")
        assert_close(f32(m), om, MASS_ATOL, MASS_RTOL, f"mass w={window}")
        assert_close(f32(ph), _per_qhead(oph), MASS_ATOL, MASS_RTOL, f"per-head w={window}")
    # w = 0: each head's mass sums to S (every probability counted once)
    np.testing.assert_allclose(f32(ph).sum(-1), w.S, rtol=1e-4)


@pytest.mark.parametrize("agg", ["sum", "mean", "max"])
@pytest.mark.parametrize("count_normalize", [False, True])
@pytest.mark.parametrize("lookahead", [-1, 0, 37])
def test_variants(kv, agg, count_normalize, lookahead):
    B, Hq, Hkv, S, D, window = 2, 8, 2, 700, 64, 21
    q = synth.bf16(synth.normal((B, Hq, S, D), 11)).cuda()
    k = synth.bf16(synth.normal((B, Hkv, S, D), 12)).cuda()
    lse, m, ph = _run(kv, q, k, window, agg=agg, count_normalize=count_normalize,
                      lookahead=lookahead)
    olse, om, oph = _full_oracle(q, k, window, agg=agg, count_normalize=count_normalize,
                                 lookahead=lookahead)
    assert_close(f32(lse), olse, LSE_ATOL, 0, "lse")
    assert_close(f32(m), om, MASS_ATOL, MASS_RTOL, "mass")
    assert_close(f32(ph), _per_qhead(oph), MASS_ATOL, MASS_RTOL, "per-head")


@pytest.mark.parametrize("B,Hq,Hkv,S,D,window", [
    (1, 1, 1, 1, 64, 0), (1, 2, 2, 31, 128, 3), (1, 4, 1, 257, 128, 255), (2, 8, 1, 333, 64, 1),
    (1, 16, 2, 513, 128, 600), (1, 2, 1, 1000, 128, 999), (1, 128, 1, 130, 64, 7),
    (3, 4, 4, 1201, 128, 64)])
def test_ragged_and_degenerate_shapes(kv, B, Hq, Hkv, S, D, window):
    q = synth.bf16(synth.normal((B, Hq, S, D), S)).cuda()
    k = synth.bf16(synth.normal((B, Hkv, S, D), S + 1)).cuda()
    lse, m, ph = _run(kv, q, k, window)
    olse, om, oph = _full_oracle(q, k, window)
    assert_close(f32(lse), olse, LSE_ATOL, 0, "lse")
    assert_close(f32(m), om, MASS_ATOL, MASS_RTOL, "mass")
    assert_close(f32(ph), _per_qhead(oph), MASS_ATOL, MASS_RTOL, "per-head")
    if window >= S:
        assert not f32(m).any()


@pytest.mark.parametrize("agg,lookahead,count_normalize", [("sum", -1, False), ("max", 300, True)])
def test_many_keys_launch_full_parity(kv, agg, lookahead, count_normalize):
    """B*Hkv*S = 67584 keys over 33 (b, KV head) pairs and three query
    chunks; every key compared with the oracle."""
    B, Hq, Hkv, S, D, window = 11, 6, 3, 2048, 64, 100
    q = synth.bf16(synth.normal((B, Hq, S, D), 21)).cuda()
    k = synth.bf16(synth.normal((B, Hkv, S, D), 22)).cuda()
    lse, m, ph = _run(kv, q, k, window, agg=agg, lookahead=lookahead,
                      count_normalize=count_normalize)
    olse, om, oph = _full_oracle(q, k, window, agg=agg, lookahead=lookahead,
                                 count_normalize=count_normalize)
    assert_close(f32(lse), olse, LSE_ATOL, 0, "lse")
    assert_close(f32(m), om, MASS_ATOL, MASS_RTOL, "mass")
    assert_close(f32(ph), _per_qhead(oph), MASS_ATOL, MASS_RTOL, "per-head")


def test_deterministic(kv):
    w = synth.QWEN4B
    q, k, _ = synth.attention_inputs(w, seed=3, device="cuda")
    a = _run(kv, q, k, w.window)
    b = _run(kv, q, k, w.window)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_qwen4b_layer(kv):
    """Qwen3-4B-shaped layer at full size: two KV-head groups compared key by
    key, sampled normalizer rows over all heads, and the w = 0 invariant."""
    w = synth.QWEN4B
    q, k, _ = synth.attention_inputs(w, seed=7, device="cuda")
    lse, m, ph = _run(kv, q, k, w.window)
    G = w.Hq // w.Hkv
    for h in (0, 5):
        olse, om, oph = oracle_group_target(q, k, 0, h, w.window, 0, w.S, all_rows=True)
        assert_close(f32(lse[0, h * G:(h + 1) * G]), olse, LSE_ATOL, 0, f"lse group {h}")
        assert_close(f32(m[0, h]), om, MASS_ATOL, MASS_RTOL, f"mass group {h}")
        assert_close(f32(ph[0, h * G:(h + 1) * G]).T, oph, MASS_ATOL, MASS_RTOL, f"per-head {h}")
    _sampled_lse_rows(q, k, lse, n=96, seed=1)
    _zero_window_invariant(kv, q, k)


def test_skewed_long_context(kv):
    """Skewed workload (B=4, S=16384, planted heavy hitters): sampled rows,
    the tail keys of two groups key by key, and the w = 0 invariant."""
    w = synth.SKEWED
    q, k, _ = synth.attention_inputs(w, seed=5, device="cuda")
    lse, m, ph = _run(kv, q, k, w.window)
    G = w.Hq // w.Hkv
    for b, h in ((0, 0), (3, 6)):
        t_lo, t_hi = w.S - w.window - 200, w.S - w.window + 8
        olse, om, oph = oracle_group_target(q, k, b, h, w.window, t_lo, t_hi)
        assert_close(f32(m[b, h, t_lo:t_hi]), om, MASS_ATOL, MASS_RTOL, f"mass ({b},{h}) tail")
        d_lo = t_lo + w.window
        assert_close(f32(lse[b, h * G:(h + 1) * G, d_lo:]), olse[:, d_lo:], LSE_ATOL, 0, "lse tail")
    _sampled_lse_rows(q, k, lse, n=64, seed=2)
    _zero_window_invariant(kv, q, k)


def test_qwen8b_prefill_layer(kv):
    """One layer of the Qwen3-8B-shaped prefill (S=32768) at full size:
    sampled normalizer rows, tail keys of one group, the w = 0 invariant."""
    w = synth.QWEN8B
    q, k, _ = synth.attention_inputs(w, seed=1000 * 4 + 17, device="cuda")
    lse, m, ph = _run(kv, q, k, w.window)
    t_lo, t_hi = w.S - w.window - 96, w.S
    olse, om, oph = oracle_group_target(q, k, 0, 3, w.window, t_lo, t_hi)
    assert_close(f32(m[0, 3, t_lo:t_hi]), om, MASS_ATOL, MASS_RTOL, "mass tail")
    _sampled_lse_rows(q, k, lse, n=24, seed=3)
    _zero_window_invariant(kv, q, k)


@pytest.mark.parametrize("wl,per_qhead", [("skewed", False), ("qwen8b", False), ("qwen8b", True)])
def test_full_size_transposed_pass_sampled_keys(kv, wl, per_qhead):
    """The transposed pass alone at full size (one run per workgroup, four
    waves of 64 keys), on one seeded normalizer array handed to both sides:
    keys at the start (summed over every query chunk), across a key-block
    boundary, one whole 256-key block (every wave and 32-key sub-tile of
    it), mid-sequence and at the tail, for the first and the last (b, KV
    head)."""
    w = synth.SKEWED if wl == "skewed" else synth.QWEN8B
    q, k, _ = synth.attention_inputs(w, seed=31, device="cuda")
    lse = synth.normalizers(w.B, w.Hq, w.S, seed=32).cuda()
    out = kv.future_attn_target(q, k, lse, w.window, per_qhead=per_qhead)
    m, ph = out if per_qhead else (out, None)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    keys = np.concatenate([np.arange(0, 24), np.arange(1010, 1040), np.arange(w.S // 2 - 12, w.S // 2 + 12),
                           np.arange(w.S // 4, w.S // 4 + 256),
                           np.arange(w.S - w.window - 24, w.S)]).astype(np.int64)
    lse_h = lse.cpu().numpy()
    for b, h in ((0, 0), (w.B - 1, w.Hkv - 1)):
        qs, ks = group_problem(q, k, b, h)
        om, oph = oracle.future_mass(qs, ks, lse_h[b:b + 1, h * G:(h + 1) * G], w.window, cols=keys,
                                     per_head=True)
        assert_close(f32(m[b, h])[keys], om, MASS_ATOL, MASS_RTOL, f"mass ({b},{h})")
        if per_qhead:
            assert_close(f32(ph[b, h * G:(h + 1) * G])[:, keys].T, oph, MASS_ATOL, MASS_RTOL,
                         f"per-head ({b},{h})")


def test_many_rows_one_run_per_workgroup_max_lookahead(kv):
    """384 (b, KV head) rows of S = 4096 at D = 128 make enough runs for one
    run per workgroup (the four-wave 64-key kernel; per-head sums at two waves
    per SIMD): MAX over the group with a 512-query lookahead and count
    normalisation, on one seeded normalizer array handed to both sides.  Keys
    at the start, across key blocks, mid-row and at the tail (where the
    lookahead and the sequence end cut the query range) of the first and the
    last row."""
    B, Hq, Hkv, S, D, window, la = 48, 32, 8, 4096, 128, 256, 512
    G = Hq // Hkv
    q = synth.bf16(synth.normal((B, Hq, S, D), 41, "cuda"))
    k = synth.bf16(synth.normal((B, Hkv, S, D), 42, "cuda"))
    lse = synth.normalizers(B, Hq, S, seed=43, device="cuda")
    m, ph = kv.future_attn_target(q, k, lse, window, lookahead=la, agg="max", count_normalize=True,
                                  per_qhead=True)
    torch.cuda.synchronize()
    keys = np.concatenate([np.arange(0, 40), np.arange(240, 300), np.arange(S // 2 - 16, S // 2 + 16),
                           np.arange(S - window - la - 40, S)]).astype(np.int64)
    lse_h = lse.cpu().numpy()
    for b, h in ((0, 0), (B - 1, Hkv - 1)):
        qs, ks = group_problem(q, k, b, h)
        om, oph = oracle.future_mass(qs, ks, lse_h[b:b + 1, h * G:(h + 1) * G], window, lookahead=la,
                                     agg="max", count_normalize=True, cols=keys, per_head=True)
        assert_close(f32(m[b, h])[keys], om, MASS_ATOL, MASS_RTOL, f"mass ({b},{h})")
        assert_close(f32(ph[b, h * G:(h + 1) * G])[:, keys].T, oph, MASS_ATOL, MASS_RTOL,
                     f"per-head ({b},{h})")


def _sampled_lse_rows(q, k, lse, n, seed):
    B, Hq, S, _ = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    r = np.random.default_rng(seed)
    picks = [(int(r.integers(B)), int(r.integers(Hq)), int(d)) for d in
             np.concatenate([r.integers(0, S, n - 4), [0, 1, S - 2, S - 1]])]
    for b, g, d in picks:
        qs, ks = group_problem(q, k, b, g // G)
        ref = oracle.lse(qs, ks, rows=np.array([(g % G) * S + d]))[0]
        got = float(lse[b, g, d])
        assert abs(got - ref) <= LSE_ATOL, (b, g, d, got, ref)


def _zero_window_invariant(kv, q, k):
    B, Hq, S, _ = q.shape
    Hkv = k.shape[1]
    lse = kv.fwd_lse(q, k)
    m = kv.future_attn_target(q, k, lse, 0)
    tot = m.double().sum(-1).cpu().numpy()
    np.testing.assert_allclose(tot, (Hq // Hkv) * S, rtol=1e-3)
