"""GPU parity of the sparse-normalizer target path (kvpop_running_topk,
kvpop_fwd_lse_sparse, then kvpop_future_attn_target on the sparse LSE)
against the CPU oracle, through the C ABI.

KVpop summary (arXiv 2607.05061v2, paperlayer.ai): App. C.1 (running top-k
mask: sinks, protected window, top-k of the eligible pool at every query),
App. C.2 (running cutoffs), Sec. 3 / App. B.3 (per-head decay as static
priorities), App. D.3 (the target reuses the sparse attention's normalizer),
App. F (fp32 ranking).

keep_until and cutoff are integer outputs of an fp32 ranking that both sides
take in fp32: they must match bit for bit.  The sparse LSE has the dense
pass's tolerance (|err| <= 1e-3) and the target mass on top of it
(|err| <= 1e-5 + 2e-3 |ref|).  The sparse pass runs in both of its modes:
listed (the budget is given: each block of queries walks the keys still
retained at its first query) and tested (every causal key is read and
tested); a listed call whose lists overflow (keep_until not made with that
budget) must still give the exact set's normalizers.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import LSE_ATOL, MASS_ATOL, MASS_RTOL, assert_close, ensure_built, f32
from oracle import brute

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    return ensure_built()


def _topk(kv, sc, s, w, budget, lam=None):
    ld = None if lam is None else torch.as_tensor(lam, dtype=torch.float32).cuda()
    u, c = kv.running_topk(sc.cuda(), s, w, budget, log_decay=ld)
    torch.cuda.synchronize()
    ou, oc = oracle.running_topk(sc.numpy(), s, w, budget,
                                 log_decay=None if lam is None else np.asarray(lam, np.float32))
    return u.cpu().numpy(), c.cpu().numpy(), ou, oc


@pytest.mark.parametrize("kind", ["normal", "ties", "special", "const", "ramp", "nan"])
@pytest.mark.parametrize("S,s,w,budget", [(256, 4, 16, 64), (1000, 4, 128, 300), (333, 70, 20, 95),
                                          (129, 0, 0, 10), (150, 2, 3, 6), (100, 4, 16, 20),
                                          (40, 4, 64, 80), (2048, 4, 128, 1024)])
def test_running_topk_bit_exact(kv, kind, S, s, w, budget):
    sc = synth.scores((2, 3, S), seed=S * 3 + budget, kind=kind)
    for lam in (None, [0.0, 0.01, 0.5]):
        u, c, ou, oc = _topk(kv, sc, s, w, budget, lam)
        assert np.array_equal(u, ou), f"keep_until differs ({kind}, lam={lam})"
        assert np.array_equal(c, oc), f"cutoff differs ({kind}, lam={lam})"


def test_running_topk_edge_cases(kv):
    sc = synth.scores((1, 2, 300), seed=9)
    for s, w, budget in ((2, 8, 10), (0, 0, 1), (4, 300, 304), (300, 0, 300), (5, 0, 64)):
        u, c, ou, oc = _topk(kv, sc, s, w, budget)
        assert np.array_equal(u, ou), (s, w, budget)
        assert np.array_equal(c, oc), (s, w, budget)
    # cutoff is optional
    u2, none = kv.running_topk(sc.cuda(), 4, 16, 64, want_cutoff=False)
    assert none is None
    assert np.array_equal(u2.cpu().numpy(), oracle.running_topk(sc.numpy(), 4, 16, 64)[0])


@pytest.mark.parametrize("S,budget,w", [(4096, 1024, 128), (32768, 8192, 256)])
def test_running_topk_full_size(kv, S, budget, w):
    """The layer (4k, budget 1024) and 32k-prefill (budget 8192) shapes: 8 KV
    heads of MLP-like scores, with a decay on half of the heads."""
    sc = synth.scores((1, 8, S), seed=S + 1)
    lam = [0.0, 1e-4, 0.0, 1e-3, 0.0, 1e-5, 0.0, 3e-4]
    u, c, ou, oc = _topk(kv, sc, 4, w, budget, lam)
    assert np.array_equal(u, ou)
    assert np.array_equal(c, oc)
    # the mask never holds more than the budget at any query
    d = np.arange(S)
    for h in range(8):
        starts = np.zeros(S + 1, np.int64)
        np.add.at(starts, np.arange(S), 1)
        np.add.at(starts, np.minimum(u[0, h], S), -1)
        live = np.cumsum(starts)[:S]  # tokens t <= d < keep_until[t]
        assert (live <= budget).all() and (live[budget - 1:] == np.minimum(d[budget - 1:] + 1, budget)).all()


@pytest.mark.parametrize("S,budget,w,s", [(40000, 5000, 256, 4), (65536, 6000, 128, 70),
                                          (33000, 300, 16, 0), (65600, 4000, 64, 4),
                                          (100000, 9000, 256, 4), (131072, 8192, 256, 130),
                                          (300000, 20000, 512, 4), (8193, 1000, 64, 4),
                                          (40000, 37000, 256, 4)])
def test_running_topk_longest_rows(kv, S, budget, w, s):
    """Rows past 8192 tokens take the sort + wavelet-matrix kernel: rank
    structures past LDS (S > 38912), the shortest such row, a budget above
    most of the row; a small budget makes most tokens leave early, a large
    one keeps many to the end."""
    sc = synth.scores((1, 2, S), seed=S + budget, kind="ties" if S == 33000 else "normal")
    u, c, ou, oc = _topk(kv, sc, s, w, budget, [0.0, 2e-5])
    assert np.array_equal(u, ou)
    assert np.array_equal(c, oc)


def test_running_topk_rejects_rows_past_its_limit(kv):
    sc = torch.zeros((1, 1, (1 << 24) + 1), dtype=torch.float32, device="cuda")
    with pytest.raises(kv.KvpopError):
        kv.running_topk(sc, 4, 16, 64)


def _sparse_oracle_rows(q, k, sc, s, w, budget, lam, rows):
    return oracle.lse_sparse(f32(q), f32(k), sc.numpy(), s, w, budget,
                             log_decay=None if lam is None else np.asarray(lam, np.float32),
                             rows=rows)


def test_tiny_sparse_target_full_parity(kv):
    """Tiny workload: running mask -> sparse LSE -> transposed pass, every
    output against the oracle (whose sparse LSE builds each query's set by
    sorting its pool)."""
    wl = synth.TINY
    q, k, _ = synth.attention_inputs(wl, seed=1)
    sc = synth.scores((wl.B, wl.Hkv, wl.S), seed=21)
    for lam, budget in ((None, 0), ([0.02], 0), (None, wl.budget), ([0.02], wl.budget)):
        ld = None if lam is None else torch.tensor(lam, dtype=torch.float32).cuda()
        u, _ = kv.running_topk(sc.cuda(), wl.n_sink, wl.window, wl.budget, log_decay=ld)
        lse = kv.fwd_lse_sparse(q.cuda(), k.cuda(), u, budget)
        mass = kv.future_attn_target(q.cuda(), k.cuda(), lse, wl.window)
        torch.cuda.synchronize()
        ol = oracle.lse_sparse(f32(q), f32(k), sc.numpy(), wl.n_sink, wl.window, wl.budget,
                               log_decay=None if lam is None else np.asarray(lam, np.float32))
        assert_close(f32(lse), ol, LSE_ATOL, 0, f"sparse lse lam={lam}")
        om = oracle.future_mass(f32(q), f32(k), ol, wl.window)
        assert_close(f32(mass), om, MASS_ATOL, MASS_RTOL, f"sparse-normalizer mass lam={lam}")
        # the dense normalizer is never smaller than the sparse one
        dense = kv.fwd_lse(q.cuda(), k.cuda())
        torch.cuda.synchronize()
        assert (f32(lse) <= f32(dense) + 1e-4).all()


@pytest.mark.parametrize("listed", [False, True])
@pytest.mark.parametrize("G,D", [(4, 128), (2, 64), (1, 128), (8, 128)])
def test_mid_size_sparse_target(kv, G, D, listed):
    """B=2, 2 KV heads, S=1100 (ragged against every tile): sparse LSE and the
    target on it, against the oracle in full."""
    wl = synth.Workload("mid", 2, 2 * G, 2, D, 1100, 64, 4, 400, rope=True, std=0.5)
    q, k, _ = synth.attention_inputs(wl, seed=G + D)
    sc = synth.scores((wl.B, wl.Hkv, wl.S), seed=G * D)
    lam = [0.0, 2e-3]
    u, _ = kv.running_topk(sc.cuda(), wl.n_sink, wl.window, wl.budget,
                           log_decay=torch.tensor(lam, dtype=torch.float32).cuda())
    lse = kv.fwd_lse_sparse(q.cuda(), k.cuda(), u, wl.budget if listed else 0)
    mass = kv.future_attn_target(q.cuda(), k.cuda(), lse, wl.window)
    torch.cuda.synchronize()
    ol = oracle.lse_sparse(f32(q), f32(k), sc.numpy(), wl.n_sink, wl.window, wl.budget,
                           log_decay=np.asarray(lam, np.float32))
    assert_close(f32(lse), ol, LSE_ATOL, 0, "sparse lse")
    om = oracle.future_mass(f32(q), f32(k), ol, wl.window)
    assert_close(f32(mass), om, MASS_ATOL, MASS_RTOL, "sparse-normalizer mass")


def test_layer_shape_sparse_lse_sampled_rows(kv):
    """The Qwen3-4B layer shape (32 q / 8 KV heads, S=4096, budget 1024, RoPE),
    in the launch the bench times: sampled rows of every head against the
    oracle, which builds each sampled query's retained set afresh."""
    wl = synth.QWEN4B
    q, k, _ = synth.attention_inputs(wl, seed=7, device="cuda")
    sc = synth.scores((wl.B, wl.Hkv, wl.S), seed=77)
    u, _ = kv.running_topk(sc.cuda(), wl.n_sink, wl.window, wl.budget)
    lse = kv.fwd_lse_sparse(q, k, u, wl.budget)
    tested = kv.fwd_lse_sparse(q, k, u)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    d = np.concatenate([[0, 1, wl.budget - 1, wl.budget, wl.S - 1], rng.integers(0, wl.S, 27)])
    rows = np.array([g * wl.S + x for g in range(wl.Hq) for x in d], np.int64)
    ref = _sparse_oracle_rows(q.cpu(), k.cpu(), sc, wl.n_sink, wl.window, wl.budget, None, rows)
    assert_close(f32(lse).reshape(-1)[rows], ref, LSE_ATOL, 0, "sparse lse rows (listed)")
    assert_close(f32(tested).reshape(-1)[rows], ref, LSE_ATOL, 0, "sparse lse rows (tested)")
    # every row: the two modes sum the same set in a different order
    assert_close(f32(lse), f32(tested), LSE_ATOL, 0, "listed against tested, all rows")


def test_prefill_shape_listed_sparse_lse_sampled_rows(kv):
    """The 32k-prefill layer shape (32 q / 8 KV heads, S = 32768, budget
    8192, RoPE) in the listed launch the bench times (lists of up to 8256
    keys per block of 32 queries): sampled rows of every head against the
    oracle, and every row against the tested mode."""
    wl = synth.QWEN8B
    q, k, _ = synth.attention_inputs(wl, seed=9, device="cuda")
    sc = synth.scores((wl.B, wl.Hkv, wl.S), seed=99)
    lam = torch.tensor([0.0, 1e-5, 0.0, 1e-4, 0.0, 3e-5, 0.0, 2e-4], dtype=torch.float32)
    u, _ = kv.running_topk(sc.cuda(), wl.n_sink, wl.window, wl.budget, log_decay=lam.cuda())
    lse = kv.fwd_lse_sparse(q, k, u, wl.budget)
    tested = kv.fwd_lse_sparse(q, k, u)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    d = np.concatenate([[0, wl.budget - 1, wl.budget, wl.budget + 31, wl.S - 1],
                        rng.integers(0, wl.S, 7)])
    rows = np.array([g * wl.S + x for g in range(wl.Hq) for x in d], np.int64)
    ref = _sparse_oracle_rows(q.cpu(), k.cpu(), sc, wl.n_sink, wl.window, wl.budget,
                              lam.numpy(), rows)
    assert_close(f32(lse).reshape(-1)[rows], ref, LSE_ATOL, 0, "32k sparse lse rows (listed)")
    assert_close(f32(lse), f32(tested), LSE_ATOL, 0, "32k listed against tested, all rows")


@pytest.mark.parametrize("B,Hq,Hkv,S", [(64, 16, 16, 500), (16, 32, 8, 1000)])
def test_many_row_blocks_full_parity(kv, B, Hq, Hkv, S):
    """Launches of many rounds of row blocks (the dense pass then keeps two
    query groups of 32 rows per wave), groups of 1 and 4, ragged last
    blocks: every dense normalizer and every sparse one (each causal key
    tested against keep_until) against the oracle."""
    D = 128
    q = synth.bf16(synth.normal((B, Hq, S, D), S + Hq))
    k = synth.bf16(synth.normal((B, Hkv, S, D), S + Hq + 1))
    sc = synth.scores((B, Hkv, S), seed=S, kind="normal")
    s, w, budget = 4, 32, 128
    qd, kd = q.cuda(), k.cuda()
    u, _ = kv.running_topk(sc.cuda(), s, w, budget)
    lse = kv.fwd_lse(qd, kd)
    lsm = kv.fwd_lse_sparse(qd, kd, u)
    torch.cuda.synchronize()
    assert_close(f32(lse), oracle.lse(f32(q), f32(k)), LSE_ATOL, 0, "dense lse")
    assert_close(f32(lsm), oracle.lse_sparse(f32(q), f32(k), sc.numpy(), s, w, budget), LSE_ATOL, 0,
                 "sparse lse")


def test_sparse_equals_dense_when_nothing_is_evicted(kv):
    """A budget covering the whole sequence keeps every key: the sparse pass
    must give the dense pass's normalizers."""
    wl = synth.Workload("noevict", 1, 8, 2, 128, 700, 32, 4, 800, rope=False, std=1.0)
    q, k, _ = synth.attention_inputs(wl, seed=4, device="cuda")
    sc = synth.scores((1, 2, wl.S), seed=5, device="cuda")
    u, _ = kv.running_topk(sc, wl.n_sink, wl.window, wl.budget)
    a = kv.fwd_lse_sparse(q, k, u)
    b = kv.fwd_lse(q, k)
    c = kv.fwd_lse_sparse(q, k, u, wl.budget)
    torch.cuda.synchronize()
    assert (u.cpu().numpy() == wl.S).all()
    assert torch.equal(a, b)
    assert_close(f32(c), f32(b), LSE_ATOL, 0, "listed, nothing evicted")


def _arbitrary_until(B, H, S, seed, kind):
    """keep_until arrays that no running top-k of a small budget makes."""
    rng = np.random.default_rng(seed)
    t = np.arange(S)
    if kind == "uniform":  # each key leaves at a random later query
        u = t + 1 + (rng.random((B, H, S)) * (S - t)).astype(np.int64)
    elif kind == "mass_exit":  # most keys leave together inside one query block
        u = np.broadcast_to(np.where(t < S // 2, S // 2 + 3, S), (B, H, S)).copy()
        u[..., :4] = S
    else:  # keys never retained or retained at their own query only: empty rows
        u = rng.integers(0, 3, (B, H, S)) + t - 1
        u[..., 100::5] = S
    return np.clip(u, 0, S).astype(np.int32)


@pytest.mark.parametrize("kind", ["uniform", "mass_exit", "empty_rows"])
@pytest.mark.parametrize("budget", [0, 24, 200, 100000])
def test_sparse_lse_any_keep_until(kv, kind, budget):
    """keep_until not made by the running top-k (and budgets that do not
    bound it): blocks whose list overflows walk their whole causal row, the
    others their list; every row must be the LSE over {t <= d < keep_until[t]}
    (brute force over the explicit membership mask; -inf for an empty set)."""
    wl = synth.Workload("any", 1, 4, 2, 128, 650, 16, 4, 64, rope=False, std=1.0)
    q, k, _ = synth.attention_inputs(wl, seed=31)
    u = _arbitrary_until(1, 2, wl.S, 5, kind)
    got = kv.fwd_lse_sparse(q.cuda(), k.cuda(), torch.from_numpy(u).cuda(), budget)
    torch.cuda.synchronize()
    d = np.arange(wl.S)
    member = (d[None, None, None, :] <= d[None, None, :, None]) & (d[None, None, :, None] < u[:, :, None, :])
    ref = brute.lse_masked(f32(q), f32(k), member)
    g = f32(got)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), "empty rows"
    fin = np.isfinite(ref)
    assert_close(g[fin], ref[fin], LSE_ATOL, 0, f"lse over any keep_until ({kind}, budget {budget})")


@pytest.mark.parametrize("S", [1, 2, 63, 65, 130])
@pytest.mark.parametrize("budget", [0, 8, 1000])
def test_sparse_lse_short_rows(kv, S, budget):
    """Sequences shorter than one key tile or one query block, and just past
    them (G = 4, P = 32), in both modes, against brute force."""
    wl = synth.Workload("short", 1, 8, 2, 64, S, 4, 1, 8, rope=False, std=1.0)
    q, k, _ = synth.attention_inputs(wl, seed=S)
    u = _arbitrary_until(1, 2, S, S + 1, "uniform")
    got = kv.fwd_lse_sparse(q.cuda(), k.cuda(), torch.from_numpy(u).cuda(), budget)
    torch.cuda.synchronize()
    d = np.arange(S)
    member = (d[None, None, None, :] <= d[None, None, :, None]) & (d[None, None, :, None] < u[:, :, None, :])
    ref = brute.lse_masked(f32(q), f32(k), member)
    g = f32(got)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert_close(g[fin], ref[fin], LSE_ATOL, 0, f"short rows S={S} budget={budget}")


def test_sparse_abi_errors(kv):
    import ctypes
    L = kv.lib()
    sc = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    u = torch.zeros((1, 1, 64), dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(sc.data_ptr())
    pu = ctypes.c_void_p(u.data_ptr())
    assert L.kvpop_running_topk(1, 1, 64, 4, 16, 10, p, None, pu, None, None, 0, None) == 1  # budget < s + w
    assert L.kvpop_running_topk(1, 1, 64, 4, 16, 30, None, None, pu, None, None, 0, None) == 1
    assert L.kvpop_running_topk(0, 1, 64, 4, 16, 30, p, None, pu, None, None, 0, None) == 1
    d = kv.dims(1, 2, 1, 64, 96)
    assert L.kvpop_fwd_lse_sparse(ctypes.byref(d), p, p, None, pu, 0, p, None, 0, None, 0, None) == 2  # D = 96
    d = kv.dims(1, 2, 1, 64, 64)
    assert L.kvpop_fwd_lse_sparse(ctypes.byref(d), p, p, None, None, 0, p, None, 0, None, 0, None) == 1
    assert L.kvpop_fwd_lse_sparse(ctypes.byref(d), p, p, None, pu, 16, p, None, 0, None, 0, None) == 1  # no workspace
