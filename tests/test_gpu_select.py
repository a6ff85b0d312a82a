"""GPU parity of retention (kvpop_evict_select: selection, slot layout,
compaction) against the oracle, bit for bit, through the C ABI.

KVpop summary: Sec. 3 (sinks + protected window + per-head top-k; attention
over the retained set only), App. C.1 (B = s + w + k), App. F (ranking and
selection in fp32).  Both sides rank the same seeded fp32 score arrays.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import MASS_ATOL, MASS_RTOL, bits, ensure_built, f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    return ensure_built()


def _compare(kv, scores, s, w, budget, D=0, seed=0):
    B, Hkv, S = scores.shape
    k = v = None
    if D:
        k = synth.bf16(synth.normal((B, Hkv, S, D), seed + 1)).cuda()
        v = synth.bf16(synth.normal((B, Hkv, S, D), seed + 2)).cuda()
    sp, ss, kc, vc = kv.evict_select(scores.cuda(), s, w, budget, k, v)
    torch.cuda.synchronize()
    osp, oss = oracle.select(f32(scores), s, w, budget)
    assert np.array_equal(sp.cpu().numpy(), osp), "slot_pos differs"
    assert np.array_equal(ss.cpu().numpy().view(np.uint32), oss.view(np.uint32)), "slot_score differs"
    if D:
        assert np.array_equal(bits(kc), oracle.gather(bits(k), osp)), "k cache differs"
        assert np.array_equal(bits(vc), oracle.gather(bits(v), osp)), "v cache differs"
    return sp


KINDS = ["normal", "ties", "special", "const", "ramp", "nan"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("name", ["tiny", "qwen3-4b-layer", "skewed-long", "qwen3-8b-prefill"])
def test_workload_shapes(kv, kind, name):
    w = synth.WORKLOADS[name]
    scores = synth.scores((w.B, w.Hkv, w.S), seed=100 * KINDS.index(kind) + len(name), kind=kind)
    _compare(kv, scores, w.n_sink, w.window, w.budget, D=w.D)


@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
def test_decode_prefix_shape(kv, kind):
    """64 sequences x 8 KV heads, prefix 32768 -> budget 4096 (512 rows)."""
    w = synth.DECODE
    scores = synth.scores((w.B, w.Hkv, w.S), seed=99, kind=kind)
    _compare(kv, scores, w.n_sink, w.window, w.budget)


@pytest.mark.parametrize("S,s,w,budget", [
    (1, 4, 16, 64), (3, 2, 4, 8), (20, 4, 16, 64), (100, 0, 0, 10), (100, 5, 0, 5),
    (100, 0, 7, 7), (5000, 4, 128, 132), (9000, 4, 1, 8200), (8193, 1, 1, 8192),
    (70000, 4, 256, 10000), (33028, 4, 256, 4096), (33029, 4, 256, 4096),
    (8452, 4, 256, 1000), (8453, 4, 256, 1000), (4228, 4, 128, 1000), (4229, 4, 128, 1000),
    (16644, 4, 256, 2000), (16645, 4, 256, 2000)])
def test_edges(kv, S, s, w, budget):
    # eligible counts on both sides of each register-path size (4K, 8K, 16K,
    # 32K per row) and beyond it; 'nan' and 'const' make every key tie
    for kind in ("normal", "ties", "special", "nan", "const"):
        scores = synth.scores((2, 3, S), seed=S + budget, kind=kind)
        _compare(kv, scores, s, w, budget, D=128 if S < 10000 else 0, seed=S)


@pytest.mark.parametrize("B,Hkv,S,s,w,budget,D", [(24, 8, 2000, 4, 64, 300, 64),
                                                   (40, 8, 700, 2, 16, 100, 128),
                                                   (1, 1, 5000, 4, 128, 1024, 128),
                                                   (1, 2, 33000, 4, 256, 8192, 64)])
def test_many_and_few_rows_with_compaction(kv, B, Hkv, S, s, w, budget, D):
    """Selection with compaction when the rows are many (one workgroup per
    row, compaction in a second launch) and few (every row selected by
    several workgroups, each compacting a share of its slots)."""
    for kind in ("normal", "ties"):
        scores = synth.scores((B, Hkv, S), seed=B + S + budget, kind=kind)
        _compare(kv, scores, s, w, budget, D=D, seed=S)


def test_deterministic(kv):
    w = synth.QWEN8B
    scores = synth.scores((w.B, w.Hkv, w.S), seed=5, kind="ties").cuda()
    a = kv.evict_select(scores, w.n_sink, w.window, w.budget)
    b = kv.evict_select(scores, w.n_sink, w.window, w.budget)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_end_to_end_from_target(kv):
    """Oracle mass -> oracle selection vs GPU mass -> GPU selection on the
    tiny and Qwen3-4B layer workloads.  The float targets agree only within
    tolerance, so a kept token may differ only where its oracle score lies
    within that tolerance of the oracle's k-th best score."""
    for w, seed in ((synth.TINY, 1), (synth.QWEN4B, 2)):
        q, k, _ = synth.attention_inputs(w, seed=seed)
        qd, kd = q.cuda(), k.cuda()
        m = kv.future_attn_target(qd, kd, kv.fwd_lse(qd, kd), w.window)
        sp, _, _, _ = kv.evict_select(m, w.n_sink, w.window, w.budget)
        h_list = range(w.Hkv) if w.Hkv <= 2 else (0, w.Hkv - 1)
        for h in h_list:
            G = w.Hq // w.Hkv
            qs, ks = f32(q[0, h * G:(h + 1) * G])[None], f32(k[0, h])[None, None]
            olse = oracle.lse(qs, ks)
            om = oracle.future_mass(qs, ks, olse, w.window)
            osp, _ = oracle.select(om.astype(np.float32), w.n_sink, w.window, w.budget)
            got = set(sp[0, h].cpu().numpy().tolist()) - {-1}
            ref = set(osp[0, 0].tolist()) - {-1}
            diff = got ^ ref
            if diff:
                kk = w.budget - w.n_sink - w.window
                elig = om[0, 0, w.n_sink:w.S - w.window]
                kth = np.sort(elig)[::-1][kk - 1]
                for t in diff:
                    assert abs(om[0, 0, t] - kth) <= MASS_ATOL + MASS_RTOL * abs(kth) * 2, (h, t)
