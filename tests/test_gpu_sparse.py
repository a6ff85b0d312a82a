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
(|err| <= 1e-5 + 2e-3 |ref|).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import LSE_ATOL, MASS_ATOL, MASS_RTOL, assert_close, ensure_built, f32

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
                                          (33000, 300, 16, 0)])
def test_running_topk_longest_rows(kv, S, budget, w, s):
    """Rows past 32768 positions take 16 segment waves per token block (the
    longest rows the kernel takes are 65536); a small budget makes most
    tokens leave early, a large one keeps many to the end."""
    sc = synth.scores((1, 2, S), seed=S + budget, kind="ties" if S == 33000 else "normal")
    u, c, ou, oc = _topk(kv, sc, s, w, budget, [0.0, 2e-5])
    assert np.array_equal(u, ou)
    assert np.array_equal(c, oc)


def test_running_topk_rejects_rows_past_its_limit(kv):
    sc = torch.zeros((1, 1, 65537), dtype=torch.float32, device="cuda")
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
    for lam in (None, [0.02]):
        ld = None if lam is None else torch.tensor(lam, dtype=torch.float32).cuda()
        u, _ = kv.running_topk(sc.cuda(), wl.n_sink, wl.window, wl.budget, log_decay=ld)
        lse = kv.fwd_lse_sparse(q.cuda(), k.cuda(), u)
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


@pytest.mark.parametrize("G,D", [(4, 128), (2, 64), (1, 128)])
def test_mid_size_sparse_target(kv, G, D):
    """B=2, 2 KV heads, S=1100 (ragged against every tile): sparse LSE and the
    target on it, against the oracle in full."""
    wl = synth.Workload("mid", 2, 2 * G, 2, D, 1100, 64, 4, 400, rope=True, std=0.5)
    q, k, _ = synth.attention_inputs(wl, seed=G + D)
    sc = synth.scores((wl.B, wl.Hkv, wl.S), seed=G * D)
    lam = [0.0, 2e-3]
    u, _ = kv.running_topk(sc.cuda(), wl.n_sink, wl.window, wl.budget,
                           log_decay=torch.tensor(lam, dtype=torch.float32).cuda())
    lse = kv.fwd_lse_sparse(q.cuda(), k.cuda(), u)
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
    lse = kv.fwd_lse_sparse(q, k, u)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    d = np.concatenate([[0, 1, wl.budget - 1, wl.budget, wl.S - 1], rng.integers(0, wl.S, 27)])
    rows = np.array([g * wl.S + x for g in range(wl.Hq) for x in d], np.int64)
    ref = _sparse_oracle_rows(q.cpu(), k.cpu(), sc, wl.n_sink, wl.window, wl.budget, None, rows)
    assert_close(f32(lse).reshape(-1)[rows], ref, LSE_ATOL, 0, "sparse lse rows")


def test_sparse_equals_dense_when_nothing_is_evicted(kv):
    """A budget covering the whole sequence keeps every key: the sparse pass
    must give the dense pass's normalizers."""
    wl = synth.Workload("noevict", 1, 8, 2, 128, 700, 32, 4, 800, rope=False, std=1.0)
    q, k, _ = synth.attention_inputs(wl, seed=4, device="cuda")
    sc = synth.scores((1, 2, wl.S), seed=5, device="cuda")
    u, _ = kv.running_topk(sc, wl.n_sink, wl.window, wl.budget)
    a = kv.fwd_lse_sparse(q, k, u)
    b = kv.fwd_lse(q, k)
    torch.cuda.synchronize()
    assert (u.cpu().numpy() == wl.S).all()
    assert torch.equal(a, b)


def test_sparse_abi_errors(kv):
    import ctypes
    L = kv.lib()
    sc = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    u = torch.zeros((1, 1, 64), dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(sc.data_ptr())
    pu = ctypes.c_void_p(u.data_ptr())
    assert L.kvpop_running_topk(1, 1, 64, 4, 16, 10, p, None, pu, None, None) == 1  # budget < s + w
    assert L.kvpop_running_topk(1, 1, 64, 4, 16, 30, None, None, pu, None, None) == 1
    assert L.kvpop_running_topk(0, 1, 64, 4, 16, 30, p, None, pu, None, None) == 1
    d = kv.dims(1, 2, 1, 64, 96)
    assert L.kvpop_fwd_lse_sparse(ctypes.byref(d), p, p, pu, p, None, 0, None) == 2  # D = 96
    d = kv.dims(1, 2, 1, 64, 64)
    assert L.kvpop_fwd_lse_sparse(ctypes.byref(d), p, p, None, p, None, 0, None) == 1
