"""GPU parity of the delayed stateful mLSTM scorer (kvpop_mlstm_step) and of
the decode step that consumes it (kvpop_cache_step with no scorer of its
own), against the CPU oracle, through the C ABI.

KVpop summary (arXiv 2607.05061v2, paperlayer.ai): App. A (running
key-value summary and normalizer), App. E.1 (input [k; v]), App. E.3 (mLSTM
matrix memory, scalar gates, stabilised form, Hedgehog features), App. E.4
(token u = q - w read out from the state through q), Sec. 3 (the token is
judged when it leaves the window).

Tolerance of a score: |gpu - oracle| <= 1e-5 + 1e-4 |oracle| (fp32 arithmetic
against the oracle's double: 256-term projections, exp/log of the gates and
a state that decays rather than grows); state entries the same, relative to
the largest entry of their row.  Keep/drop decisions and the cache layout
are compared bit for bit, with the GPU's own scores fed to the oracle's
cache step (no GPU output is an expected value).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import assert_close, bits, ensure_built, f32

pytestmark = pytest.mark.gpu

SC_ATOL, SC_RTOL = 1e-5, 1e-4
P, E = 32, 64


@pytest.fixture(scope="module")
def kv():
    return ensure_built()


def _params(H, D, seed, bi=0.0, bf=3.0):
    g = torch.Generator().manual_seed(seed)
    X = 2 * D
    r = lambda *sh: torch.randn(sh, generator=g, dtype=torch.float32)
    return {"wk": r(H, P, X) / X ** 0.5, "wr": r(H, P, X) / X ** 0.5, "wv": r(H, E, X) / X ** 0.5,
            "wi": r(H, X) / X ** 0.5, "bi": torch.full((H,), bi), "wf": r(H, X) / X ** 0.5,
            "bf": torch.full((H,), bf), "wo": r(H, E) / E ** 0.5, "bo": r(H) * 0.1}


def _tokens(B, H, n, D, seed):
    k = synth.bf16(synth.normal((B, H, n, D), seed, std=0.5))
    v = synth.bf16(synth.normal((B, H, n, D), seed + 1, std=0.5))
    return k, v


@pytest.mark.parametrize("D,bi,bf", [(128, 0.0, 3.0), (64, 0.0, 3.0), (128, 6.0, -1.0)])
def test_scores_and_state_match_the_scan(kv, D, bi, bf):
    B, H, n, s, w, budget = 2, 3, 300, 4, 16, 64
    kk = budget - s - w
    k, v = _tokens(B, H, n, D, seed=D + int(bi))
    pr = _params(H, D, seed=D, bi=bi, bf=bf)
    prd = {a: t.cuda() for a, t in pr.items()}
    kd, vd = k.cuda(), v.cuda()
    kc = torch.zeros((B, H, budget, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    ss = torch.full((B, H, budget), float("nan"), device="cuda")
    state = kv.mlstm_state(B, H)
    got = np.full((B, H, n), np.nan)
    for t in range(n):
        kv.mlstm_step(kd[:, :, t].contiguous(), vd[:, :, t].contiguous(), prd, state, t, s, w,
                      kc, vc, ss)
        u = t - w
        if u >= s:
            got[:, :, u] = ss[:, :, s + kk + u % w].cpu().numpy()
        # the token enters its ring slot after the scorer has read the exiting one
        slot = t if t < s else s + kk + t % w
        kc[:, :, slot] = kd[:, :, t]
        vc[:, :, slot] = vd[:, :, t]
    torch.cuda.synchronize()
    ref, (C, nr, m) = oracle.mlstm_scores(f32(k), f32(v), {a: t.numpy() for a, t in pr.items()}, w,
                                          want_state=True)
    sel = np.zeros((B, H, n), bool)
    sel[:, :, s:n - w] = True
    assert_close(got[sel], ref[sel], SC_ATOL, SC_RTOL, "mlstm scores")
    st = state.cpu().numpy()
    Cg = st[..., :E * 2 * P].reshape(B, H, E, 2 * P)
    scale = np.abs(C).max(axis=(2, 3), keepdims=True)
    assert (np.abs(Cg - C) <= 1e-5 * scale + 1e-4 * np.abs(C)).all(), "matrix memory"
    ng = st[..., E * 2 * P:E * 2 * P + 2 * P]
    assert (np.abs(ng - nr) <= 1e-5 * np.abs(nr).max(axis=-1, keepdims=True) + 1e-4 * np.abs(nr)).all()
    np.testing.assert_allclose(st[..., E * 2 * P + 2 * P], m, rtol=1e-5, atol=1e-5)


def test_state_update_only_leaves_scores_alone(kv):
    B, H, D = 1, 2, 128
    k, v = _tokens(B, H, 40, D, seed=3)
    prd = {a: t.cuda() for a, t in _params(H, D, seed=3).items()}
    state = kv.mlstm_state(B, H)
    for t in range(40):
        kv.mlstm_step(k[:, :, t].contiguous().cuda(), v[:, :, t].contiguous().cuda(), prd, state, t,
                      4, 16)
    torch.cuda.synchronize()
    _, (C, _, m) = oracle.mlstm_scores(f32(k), f32(v), {a: t.cpu().numpy() for a, t in prd.items()},
                                       16, want_state=True)
    st = state.cpu().numpy()
    np.testing.assert_allclose(st[..., E * 2 * P + 2 * P], m, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("fused", [False, True])
def test_decode_with_mlstm_scores_bit_exact_cache(kv, fused):
    """Decode from an empty cache: at every position the scorer takes the new
    token and scores the exiting one, then the cache step (no scorer of its
    own) keeps or drops it.  The cache after every step equals the oracle's
    cache step fed the same (GPU) scores; the scores match the oracle's scan."""
    B, H, G, D, s, w, budget, n = 2, 2, 2, 128, 4, 16, 40, 200
    kk = budget - s - w
    k, v = _tokens(B, H, n, D, seed=11)
    q = synth.bf16(synth.normal((B, H * G, n, D), 13, std=0.5))
    pr = _params(H, D, seed=12)
    prd = {a: t.cuda() for a, t in pr.items()}
    kc = torch.zeros((B, H, budget, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    sp = torch.full((B, H, budget), -1, dtype=torch.int32, device="cuda")
    ss = torch.full((B, H, budget), float("-inf"), device="cuda")
    state = kv.mlstm_state(B, H)
    ost = {"kc": bits(kc).copy(), "vc": bits(vc).copy(), "slot_pos": sp.cpu().numpy().copy(),
           "slot_score": ss.cpu().numpy().copy()}
    nan_r = np.full((B, H), np.nan, np.float32)
    got = np.full((B, H, n), np.nan)
    for t in range(n):
        kn, vn = k[:, :, t].contiguous().cuda(), v[:, :, t].contiguous().cuda()
        kv.mlstm_step(kn, vn, prd, state, t, s, w, kc, vc, ss)
        u = t - w
        if u >= s:
            ring = s + kk + u % w
            got[:, :, u] = ss[:, :, ring].cpu().numpy()
            ost["slot_score"][:, :, ring] = got[:, :, u].astype(np.float32)
        if fused:
            kv.decode_step(q[:, :, t].contiguous().cuda(), kc, vc, sp, ss, kn, vn, t, s, w, 0)
        else:
            kv.cache_step(kc, vc, sp, ss, kn, vn, t, s, w, 0)
        oracle.cache_step(ost, bits(k[:, :, t]), bits(v[:, :, t]), nan_r, s, w, 0, t)
        torch.cuda.synchronize()
        assert np.array_equal(sp.cpu().numpy(), ost["slot_pos"]), f"slot positions at step {t}"
        assert np.array_equal(bits(kc), ost["kc"]) and np.array_equal(bits(vc), ost["vc"])
        gs, os_ = ss.cpu().numpy(), ost["slot_score"]
        assert np.array_equal(np.isnan(gs), np.isnan(os_)) and np.array_equal(gs[~np.isnan(gs)], os_[~np.isnan(os_)])
    ref = oracle.mlstm_scores(f32(k), f32(v), {a: t.numpy() for a, t in pr.items()}, w)
    sel = np.zeros((B, H, n), bool)
    sel[:, :, s:n - w] = True
    assert_close(got[sel], ref[sel], SC_ATOL, SC_RTOL, "mlstm scores in decode")


@pytest.mark.parametrize("B,H,G,D,budget,pos", [(64, 8, 4, 128, 300, 5000), (2, 2, 4, 128, 300, 5000),
                                                (3, 4, 2, 64, 100, 777)])
def test_fused_decode_step_mlstm_matches_the_calls(kv, B, H, G, D, budget, pos):
    """kvpop_decode_step_mlstm = kvpop_mlstm_step + kvpop_decode_step (no
    scorer), bit for bit: state, slot positions and scores, caches, o, lse.
    The first shape takes the one-launch path, the others the split plan."""
    s, w = 4, 64
    g = torch.Generator(device="cuda").manual_seed(B + budget)
    kc = torch.randn((B, H, budget, D), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((B, H, budget, D), generator=g, device="cuda").to(torch.bfloat16)
    sp = torch.arange(budget, dtype=torch.int32, device="cuda").repeat(B, H, 1)
    sp[..., s:budget - w] = torch.randint(s, pos - w, (B, H, budget - w - s), generator=g,
                                          device="cuda", dtype=torch.int32)
    ring = [0] * w
    for p_ in range(pos - w, pos):  # token p sits in ring slot (budget - w) + p mod w
        ring[p_ % w] = p_
    sp[..., budget - w:] = torch.tensor(ring, dtype=torch.int32, device="cuda")
    ss = torch.randn((B, H, budget), generator=g, device="cuda")
    kn = torch.randn((B, H, D), generator=g, device="cuda").to(torch.bfloat16)
    vn = torch.randn((B, H, D), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, H * G, D), generator=g, device="cuda").to(torch.bfloat16)
    prd = {a: t.cuda() for a, t in _params(H, D, seed=B).items()}
    state = kv.mlstm_state(B, H)
    for t in range(5):  # a non-empty state
        kv.mlstm_step(kn, vn, prd, state, t, s, w)
    copies = [x.clone() for x in (kc, vc, sp, ss, state)]
    kv.mlstm_step(kn, vn, prd, state, pos, s, w, kc, vc, ss)
    o1, l1 = kv.decode_step(q, kc, vc, sp, ss, kn, vn, pos, s, w, 0)
    kc2, vc2, sp2, ss2, st2 = copies
    o2, l2 = kv.decode_step_mlstm(q, kc2, vc2, sp2, ss2, kn, vn, prd, st2, pos, s, w)
    torch.cuda.synchronize()
    for a, b_, name in ((kc, kc2, "k cache"), (vc, vc2, "v cache"), (sp, sp2, "slot_pos"),
                        (o1, o2, "o"), (l1, l2, "lse"), (state, st2, "state")):
        assert torch.equal(a, b_), name
    assert torch.equal(torch.nan_to_num(ss, nan=7.0), torch.nan_to_num(ss2, nan=7.0))
