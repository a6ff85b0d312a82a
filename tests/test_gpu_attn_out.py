"""GPU parity of the main pass's attention output (kvpop_fwd_lse and
kvpop_fwd_lse_sparse with v and o) against the CPU oracle, through the C ABI.

KVpop summary (arXiv 2607.05061v2, paperlayer.ai): App. D.4, first step (the
main attention pass, whose per-query normalizers the target reuses) and
App. I (the sparse student attention over the fixed-budget mask of App. C.1
supplies output and normalizers).

Tolerance of O, from the arithmetic of the pass: every probability p_dt
enters the product with V rounded to bf16 (relative error at most 2^-9),
while the normalizer sums the fp32 values, so
  |O_gpu - O| <= 2^-9 * A + (fp32 accumulation),  A[c] = sum_t p_dt |v_t[c]|
(A is the oracle's o_abs).  The bar is |O_gpu - O| <= 1e-5 + 2e-3 |O| +
2^-8 A, twice the rounding bound; a bf16 output adds one more rounding,
2^-8 |O|.  LSE |d| <= 1e-3, as for the LSE-only pass.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import LSE_ATOL, assert_close, ensure_built, f32, group_problem

pytestmark = pytest.mark.gpu

O_ATOL, O_RTOL, O_ABS = 1e-5, 2e-3, 2.0 ** -8


@pytest.fixture(scope="module")
def kv():
    return ensure_built()


def _check_o(got, ref, ref_abs, bf16_out, what):
    got = np.asarray(got, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    bound = O_ATOL + (O_RTOL + (2.0 ** -8 if bf16_out else 0.0)) * np.abs(ref) + O_ABS * ref_abs
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"got={got[i]!r} ref={ref[i]!r} err={err[i]:.3e} bound={bound[i]:.3e}")


def _inputs(B, Hq, Hkv, S, D, seed, std=1.0):
    q = synth.bf16(synth.normal((B, Hq, S, D), seed, std=std))
    k = synth.bf16(synth.normal((B, Hkv, S, D), seed + 1, std=std))
    v = synth.bf16(synth.normal((B, Hkv, S, D), seed + 2))
    return q, k, v


@pytest.mark.parametrize("B,Hq,Hkv,S,D", [(1, 2, 1, 256, 64), (1, 4, 1, 1, 128), (2, 8, 2, 130, 128),
                                          (1, 8, 8, 257, 64), (1, 16, 2, 1000, 128),
                                          (3, 4, 4, 31, 128), (1, 32, 4, 200, 64)])
def test_dense_output_full_parity(kv, B, Hq, Hkv, S, D):
    """Every row against the oracle: one row, ragged tails, groups of 1 to 8,
    both head dims and both output types."""
    q, k, v = _inputs(B, Hq, Hkv, S, D, seed=S + D + Hq)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    lse, o = kv.fwd_lse(qd, kd, v=vd)
    lse_b, ob = kv.fwd_lse(qd, kd, v=vd, out_dtype=torch.bfloat16)
    lse_only = kv.fwd_lse(qd, kd)
    torch.cuda.synchronize()
    oo, oa, ol = oracle.attn_out(f32(q), f32(k), f32(v))
    assert_close(f32(lse), ol, LSE_ATOL, 0, "lse")
    assert_close(f32(lse_only), ol, LSE_ATOL, 0, "lse (no output)")
    assert torch.equal(lse.view(torch.int32), lse_b.view(torch.int32))
    _check_o(f32(o), oo, oa, False, "o fp32")
    _check_o(f32(ob), oo, oa, True, "o bf16")


def test_tiny_workload_and_closed_forms(kv):
    """The tiny workload's inputs; then V constant per channel gives that
    constant for every row, and the first row returns v_0."""
    w = synth.TINY
    q, k, v = synth.attention_inputs(w, seed=1)
    lse, o = kv.fwd_lse(q.cuda(), k.cuda(), v=v.cuda())
    torch.cuda.synchronize()
    oo, oa, ol = oracle.attn_out(f32(q), f32(k), f32(v))
    assert_close(f32(lse), ol, LSE_ATOL, 0, "lse")
    _check_o(f32(o), oo, oa, False, "o")
    G = w.Hq // w.Hkv
    for g in range(w.Hq):
        np.testing.assert_array_equal(f32(o)[0, g, 0], f32(v)[0, g // G, 0])
    vc = torch.arange(w.D, dtype=torch.float32).sub(20.0).mul(0.125).to(torch.bfloat16)
    vc = vc.expand(w.B, w.Hkv, w.S, w.D).contiguous()
    _, oc = kv.fwd_lse(q.cuda(), k.cuda(), v=vc.cuda())
    torch.cuda.synchronize()
    ref = np.broadcast_to(f32(vc)[:, :1, :1], (w.B, w.Hq, w.S, w.D))
    # a convex combination of equal bf16 values, the weights rounded to bf16
    # and normalised by their fp32 sum: within the rounding bound of the weights
    assert (np.abs(f32(oc) - ref) <= 1e-6 + 2.0 ** -8 * np.abs(ref)).all()


@pytest.mark.parametrize("S,s,w,budget,G,D", [(256, 4, 16, 64, 2, 64), (300, 0, 8, 40, 4, 128),
                                              (130, 2, 0, 20, 1, 128), (1000, 4, 32, 200, 8, 128)])
def test_sparse_output_full_parity(kv, S, s, w, budget, G, D):
    """The sparse attention output over the running top-k mask (keep_until
    from the oracle's mask), every row against the oracle's sparse output,
    with and without a budget argument (the output mode reads every key)."""
    B, Hkv = 2, 2
    q, k, v = _inputs(B, Hkv * G, Hkv, S, D, seed=S + budget)
    sc = synth.scores((B, Hkv, S), seed=S, kind="normal")
    lds = np.array([0.0, 0.01], np.float32)
    until, _ = oracle.running_topk(sc.numpy(), s, w, budget, log_decay=lds)
    ud = torch.from_numpy(until).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    lse, o = kv.fwd_lse_sparse(qd, kd, ud, 0, v=vd)
    lse2, o2 = kv.fwd_lse_sparse(qd, kd, ud, budget, v=vd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    oo, oa, ol = oracle.attn_out(f32(q), f32(k), f32(v), sc.numpy(), s, w, budget, log_decay=lds)
    assert_close(f32(lse), ol, LSE_ATOL, 0, "sparse lse")
    assert_close(f32(lse2), ol, LSE_ATOL, 0, "sparse lse (budget given)")
    _check_o(f32(o), oo, oa, False, "sparse o")
    _check_o(f32(o2), oo, oa, True, "sparse o bf16")


def _sampled_rows(kv, w, seed, n_rows, sparse=False):
    dev = "cuda"
    q, k, v = synth.attention_inputs(w, seed=seed, device=dev)
    G = w.Hq // w.Hkv
    if sparse:
        sc = synth.scores((w.B, w.Hkv, w.S), seed=seed, device=dev)
        until, _ = kv.running_topk(sc, w.n_sink, w.window, w.budget)
        lse, o = kv.fwd_lse_sparse(q, k, until, w.budget, v=v)
    else:
        lse, o = kv.fwd_lse(q, k, v=v)
    torch.cuda.synchronize()
    r = np.random.default_rng(seed)
    picks = [(int(r.integers(w.B)), int(r.integers(w.Hq)), int(d)) for d in
             np.concatenate([r.integers(0, w.S, n_rows - 4), [0, 1, w.S - 2, w.S - 1]])]
    for b, g, d in picks:
        h = g // G
        qs, ks = group_problem(q, k, b, h)
        vs = np.ascontiguousarray(f32(v[b, h])[None, None])
        row = np.array([(g % G) * w.S + d], np.int64)
        if sparse:
            scs = np.ascontiguousarray(sc[b, h].cpu().numpy()[None, None])
            oo, oa, ol = oracle.attn_out(qs, ks, vs, scs, w.n_sink, w.window, w.budget, rows=row)
        else:
            oo, oa, ol = oracle.attn_out(qs, ks, vs, rows=row)
        assert abs(float(lse[b, g, d]) - ol[0]) <= LSE_ATOL, (b, g, d)
        _check_o(f32(o[b, g, d])[None], oo, oa, False, f"row ({b},{g},{d})")


@pytest.mark.parametrize("wl,sparse", [("qwen4b", False), ("qwen4b", True), ("qwen8b", False),
                                       ("qwen8b", True)])
def test_full_size_sampled_rows(kv, wl, sparse):
    """The 4k layer and one 32k-prefill layer at full size: sampled rows of
    every kind (first, second, last two, random) against the oracle."""
    w = synth.QWEN4B if wl == "qwen4b" else synth.QWEN8B
    print(f"attention output at {w.name} sparse={sparse}", flush=True)
    _sampled_rows(kv, w, seed=77 if wl == "qwen4b" else 78, n_rows=24 if wl == "qwen4b" else 12,
                  sparse=sparse)


def _jump_inputs(seed):
    """Queries and keys whose scores jump far past every earlier score of
    their rows: rows d >= 256 of the first query head of each group align
    with a direction u of their KV head, keys 300 and 301 carry 26 u (about
    60 above the earlier maximum, so the pass has to take its maximum
    again) and key 500 carries 34 u (about 18 above that: a term near e^18
    that the pass keeps relative to the older maximum); key 700 carries 9 u,
    below both."""
    B, Hq, Hkv, S, D = 1, 4, 2, 1000, 128
    G = Hq // Hkv
    q = synth.normal((B, Hq, S, D), seed)
    k = synth.normal((B, Hkv, S, D), seed + 1)
    v = synth.normal((B, Hkv, S, D), seed + 2)
    u = synth.normal((Hkv, D), seed + 3)
    u = u / u.norm(dim=1, keepdim=True)
    for h in range(Hkv):
        q[0, h * G, 256:] += 26.0 * u[h]
        for t, a in ((300, 26.0), (301, 26.0), (500, 34.0), (700, 9.0)):
            k[0, h, t] = a * u[h] + 0.1 * k[0, h, t]
    return synth.bf16(q), synth.bf16(k), synth.bf16(v)


def test_score_jumps_full_parity(kv):
    """Scores far above a row's earlier maximum (the pass takes the maximum
    again) and moderately above it (the pass keeps terms above 1): LSE-only,
    attention output and the sparse modes, every row against the oracle."""
    q, k, v = _jump_inputs(seed=91)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    _, Hkv, S, _ = k.shape
    sc = synth.scores((1, Hkv, S), seed=92, kind="normal")
    n_sink, window, budget = 4, 32, 200
    until, _ = oracle.running_topk(sc.numpy(), n_sink, window, budget)
    ud = torch.from_numpy(until).cuda()
    lse = kv.fwd_lse(qd, kd)
    lse_o, o = kv.fwd_lse(qd, kd, v=vd)
    lse_m = kv.fwd_lse_sparse(qd, kd, ud)
    lse_l = kv.fwd_lse_sparse(qd, kd, ud, budget)
    lse_mo, o_m = kv.fwd_lse_sparse(qd, kd, ud, 0, v=vd)
    torch.cuda.synchronize()
    oo, oa, ol = oracle.attn_out(f32(q), f32(k), f32(v))
    assert ol.max() > 50.0  # the planted scores are there
    assert_close(f32(lse), ol, LSE_ATOL, 0, "lse")
    assert_close(f32(lse_o), ol, LSE_ATOL, 0, "lse with output")
    _check_o(f32(o), oo, oa, False, "o")
    so, sa, sl = oracle.attn_out(f32(q), f32(k), f32(v), sc.numpy(), n_sink, window, budget)
    assert_close(f32(lse_m), sl, LSE_ATOL, 0, "sparse lse (every key tested)")
    assert_close(f32(lse_l), sl, LSE_ATOL, 0, "sparse lse (listed keys)")
    assert_close(f32(lse_mo), sl, LSE_ATOL, 0, "sparse lse with output")
    _check_o(f32(o_m), so, sa, False, "sparse o")
