"""Shared helpers of the GPU parity tests (no test functions here).

Tolerances (the parity bar for fp32 accumulation of bf16 inputs):
  LSE      |gpu - oracle| <= 1e-3
  mass     |gpu - oracle| <= 1e-5 + 2e-3 |oracle|
  decode o |gpu - oracle| <= 1e-5 + 2e-3 |oracle| (fp32 output);
           bf16 output adds one bf16 rounding: + 2^-8 |oracle|
  MLP      |gpu - oracle| <= 1e-5 + 1e-4 |oracle|
Indices, slot layouts and compacted caches are compared bit for bit.
"""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402

LSE_ATOL = 1e-3
MASS_ATOL, MASS_RTOL = 1e-5, 2e-3
O_ATOL, O_RTOL = 1e-5, 2e-3
MLP_ATOL, MLP_RTOL = 1e-5, 1e-4


def ensure_built():
    import future_attention_scoring_kvpop_amd as kv
    if not os.path.exists(kv.LIB_PATH):
        from future_attention_scoring_kvpop_amd import build
        build.build()
    from oracle import build as ob
    if not os.path.exists(ob.LIB):
        ob.build()
    return kv


def f32(t):
    """Exact float32 numpy copy of a (bf16 or fp32) tensor."""
    return t.detach().float().cpu().numpy()


def bits(t):
    """Raw bf16 bit patterns as uint16 numpy."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def assert_close(got, ref, atol, rtol, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finiteness differs"
    assert np.array_equal(got[~fin], ref[~fin]), f"{what}: non-finite values differ"
    err = np.abs(got[fin] - ref[fin])
    bound = atol + rtol * np.abs(ref[fin])
    bad = err > bound
    if bad.any():
        i = np.argmax(err - bound)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst "
                             f"got={got[fin][i]!r} ref={ref[fin][i]!r} err={err[i]:.3e} "
                             f"bound={bound[i]:.3e}")


def group_problem(q, k, b, h):
    """The (b, KV head h) sub-problem: B=1, Hq=G, Hkv=1 float32 arrays."""
    G = q.shape[1] // k.shape[1]
    qs = f32(q[b, h * G:(h + 1) * G])[None]
    ks = f32(k[b, h])[None, None]
    return np.ascontiguousarray(qs), np.ascontiguousarray(ks)


def oracle_group_target(q, k, b, h, window, t_lo, t_hi, lookahead=-1, agg="sum",
                        count_normalize=False, scale=None, all_rows=False):
    """Oracle LSE rows and per-key mass for keys [t_lo, t_hi) of one group.

    Only the normalizer rows those keys need (d >= t_lo + w) are computed
    unless all_rows; every other row is left NaN so an accidental read would
    show.
    Returns (lse_sub [G,S] with NaN gaps, mass [t_hi-t_lo], per_head [n,G]).
    """
    qs, ks = group_problem(q, k, b, h)
    G, S = qs.shape[1], qs.shape[2]
    d_lo = 0 if all_rows else min(S, t_lo + window)
    rows = np.array([g * S + d for g in range(G) for d in range(d_lo, S)], np.int64)
    lse_sub = np.full((1, G, S), np.nan)
    if rows.size:
        lse_sub.reshape(-1)[rows] = oracle.lse(qs, ks, scale=scale, rows=rows)
    cols = np.arange(t_lo, t_hi, dtype=np.int64)
    m, ph = oracle.future_mass(qs, ks, lse_sub, window, lookahead=lookahead, agg=agg,
                               count_normalize=count_normalize, cols=cols, per_head=True,
                               scale=scale)
    return lse_sub[0], m, ph
