"""GPU parity of the decode side (kvpop_decode_attend, kvpop_score_mlp,
kvpop_cache_step) against the oracle, through the C ABI.

KVpop summary: Sec. 3 (attention over the retained set; a token is scored
while in the window and judged when it leaves it), App. C.1 (decoding over
retained entries; B = s + w + k), App. E.2 (headwise MLP scorer), App. E.4
(u = q - w is the newly eligible token).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (MLP_ATOL, MLP_RTOL, O_ATOL, O_RTOL, assert_close, bits, ensure_built, f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    return ensure_built()


def _cache(B, Hkv, n, D, seed, empty_frac=0.2):
    kc = synth.bf16(synth.normal((B, Hkv, n, D), seed, std=0.5))
    vc = synth.bf16(synth.normal((B, Hkv, n, D), seed + 1))
    g = torch.Generator().manual_seed(seed + 2)
    sp = torch.arange(n, dtype=torch.int32).expand(B, Hkv, n).contiguous()
    sp = torch.where(torch.rand((B, Hkv, n), generator=g) < empty_frac, torch.full_like(sp, -1), sp)
    return kc, vc, sp


@pytest.mark.parametrize("B,Hq,Hkv,n,D", [(2, 8, 2, 1000, 128), (1, 4, 4, 37, 64), (3, 16, 2, 300, 128),
                                          (2, 32, 2, 5000, 64), (1, 2, 1, 64, 128), (1, 1, 1, 1, 128),
                                          (4, 32, 8, 4096, 128)])
def test_decode_attend_parity(kv, B, Hq, Hkv, n, D):
    kc, vc, sp = _cache(B, Hkv, n, D, seed=n + D)
    q = synth.bf16(synth.normal((B, Hq, D), n))
    o, lse = kv.decode_attend(q.cuda(), kc.cuda(), vc.cuda(), sp.cuda())
    ob, _ = kv.decode_attend(q.cuda(), kc.cuda(), vc.cuda(), sp.cuda(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    oo, ol = oracle.decode_attend(f32(q), f32(kc), f32(vc), sp.numpy())
    assert_close(f32(o), oo, O_ATOL, O_RTOL, "o fp32")
    assert_close(f32(lse), ol, 1e-4, 0, "lse")
    assert_close(f32(ob), oo, O_ATOL, O_RTOL + 2.0 ** -8, "o bf16")


@pytest.mark.parametrize("n", [1000, 4096])
def test_decode_attend_score_jumps(kv, n):
    """Slots whose scores rise far past every earlier slot's (the kernel has
    to take its maximum again) and a little past it (terms above 1 kept as
    they are), over a short and a long row."""
    B, Hq, Hkv, D = 2, 8, 2, 128
    G = Hq // Hkv
    kc, vc, sp = _cache(B, Hkv, n, D, seed=n + 7, empty_frac=0.1)
    q = synth.normal((B, Hq, D), n + 8)
    u = synth.normal((B, Hkv, D), n + 9)
    u = u / u.norm(dim=-1, keepdim=True)
    kf = kc.float()
    for b in range(B):
        for h in range(Hkv):
            q[b, h * G:(h + 1) * G] += 20.0 * u[b, h]
            for j, a in ((n // 3, 30.0), (n // 3 + 70, 30.0), (2 * n // 3, 38.0), (n - 5, 10.0)):
                kf[b, h, j] = a * u[b, h]
                sp[b, h, j] = j
    kc, q = synth.bf16(kf), synth.bf16(q)
    o, lse = kv.decode_attend(q.cuda(), kc.cuda(), vc.cuda(), sp.cuda())
    torch.cuda.synchronize()
    oo, ol = oracle.decode_attend(f32(q), f32(kc), f32(vc), sp.numpy())
    assert ol.max() > 50.0  # the planted scores are there
    assert_close(f32(o), oo, O_ATOL, O_RTOL, "o")
    assert_close(f32(lse), ol, 1e-4, 0, "lse")


def test_decode_workload_shape_and_empty_rows(kv):
    """64 sequences x 32/8 heads over 4096 slots, one row fully empty."""
    B, Hq, Hkv, n, D = 64, 32, 8, 4096, 128
    kc, vc, sp = _cache(B, Hkv, n, D, seed=5, empty_frac=0.05)
    sp[3, 2] = -1
    q = synth.bf16(synth.normal((B, Hq, D), 6, std=0.5))
    o, lse = kv.decode_attend(q.cuda(), kc.cuda(), vc.cuda(), sp.cuda())
    torch.cuda.synchronize()
    oo, ol = oracle.decode_attend(f32(q), f32(kc), f32(vc), sp.numpy())
    assert_close(f32(o), oo, O_ATOL, O_RTOL, "o")
    assert_close(f32(lse), ol, 1e-4, 0, "lse")
    assert not f32(o)[3, 8:12].any() and np.all(f32(lse)[3, 8:12] == -np.inf)


@pytest.mark.parametrize("B,Hkv,n,D,hidden", [(2, 8, 700, 128, 64), (3, 2, 1001, 64, 40),
                                              (1, 3, 5, 128, 1), (2, 4, 4099, 128, 17),
                                              (1, 1, 1, 64, 64)])
def test_score_mlp_parity(kv, B, Hkv, n, D, hidden):
    """Every token against the oracle: ragged runs per wave, hidden < 64
    (lanes without a unit), D = 64 and a single token."""
    keys = synth.bf16(synth.normal((B, Hkv, n, D), 3 + n, std=0.5))
    w1, b1, w2, b2 = synth.mlp_weights(Hkv, D, hidden, seed=4 + hidden)
    b1 = b1 + 0.1
    b2 = b2 - 0.3
    sc = kv.score_mlp(keys.cuda(), w1.cuda(), b1.cuda(), w2.cuda(), b2.cuda())
    torch.cuda.synchronize()
    ref = oracle.mlp_score(f32(keys), w1.numpy(), b1.numpy(), w2.numpy(), b2.numpy())
    assert_close(f32(sc), ref, MLP_ATOL, MLP_RTOL, "mlp")


def test_score_mlp_decode_prefix_sampled(kv):
    """The decode workload's prefix at full size (64 x 8 x 32768 keys, runs
    of 512 tokens per wave): sampled tokens of every row against the oracle,
    including the first and last token of each row and of a run."""
    w = synth.DECODE
    keys = synth.bf16(synth.normal((w.B, w.Hkv, w.S, w.D), 12, device="cuda", std=w.std))
    mlp = [t.cuda() for t in synth.mlp_weights(w.Hkv, w.D, w.extra["hidden"], seed=13)]
    sc = kv.score_mlp(keys, *mlp)
    torch.cuda.synchronize()
    r = np.random.default_rng(14)
    toks = np.unique(np.concatenate([[0, 511, 512, w.S - 1], r.integers(0, w.S, 28)]))
    got = f32(sc[:, :, toks])
    ref = oracle.mlp_score(f32(keys[:, :, toks]), *(t.cpu().numpy() for t in mlp))
    assert_close(got, ref, MLP_ATOL, MLP_RTOL, "mlp prefix")


def _prefix_state(kv, B, Hkv, S0, D, s, w, budget, seed):
    k = synth.bf16(synth.normal((B, Hkv, S0, D), seed, std=0.5)).cuda()
    v = synth.bf16(synth.normal((B, Hkv, S0, D), seed + 1)).cuda()
    sc = synth.scores((B, Hkv, S0), seed + 2, kind="ties").cuda()
    sp, ss, kc, vc = kv.evict_select(sc, s, w, budget, k, v)
    return {"kc": kc, "vc": vc, "slot_pos": sp, "slot_score": ss}


def _host_state(st):
    return {"kc": bits(st["kc"]).copy(), "vc": bits(st["vc"]).copy(),
            "slot_pos": st["slot_pos"].cpu().numpy().copy(),
            "slot_score": st["slot_score"].cpu().numpy().copy()}


def _same_state(g, o, what):
    assert np.array_equal(g["slot_pos"].cpu().numpy(), o["slot_pos"]), f"{what}: slot_pos"
    assert np.array_equal(g["slot_score"].cpu().numpy().view(np.uint32),
                          o["slot_score"].view(np.uint32)), f"{what}: slot_score"
    assert np.array_equal(bits(g["kc"]), o["kc"]), f"{what}: k cache"
    assert np.array_equal(bits(g["vc"]), o["vc"]), f"{what}: v cache"


@pytest.mark.parametrize("s,w,k,delay,D", [(4, 16, 40, 5, 128), (1, 8, 6, 0, 64), (0, 4, 3, 3, 128),
                                           (2, 5, 0, 2, 64), (4, 256, 3836, 16, 128),
                                           (4, 256, 5000, 16, 128)])  # > 4096 kept: multi-pass scan
def test_cache_step_bit_exact_with_given_scores(kv, s, w, k, delay, D):
    """Decisions from identical fp32 scores must match the oracle bit for bit.
    The last case keeps more long-range tokens than one pass of the step's
    worst-token scan covers (4096), so the scan runs in several passes."""
    B, Hkv = 3, 2
    budget = s + w + k
    S0 = max(2 * budget, s + w + 3)
    steps = 300 if budget < 1000 else 40
    st = _prefix_state(kv, B, Hkv, S0, D, s, w, budget, seed=budget)
    ost = _host_state(st)
    _same_state(st, ost, "prefix")
    g = torch.Generator().manual_seed(budget + 1)
    for i in range(steps):
        q = S0 + i
        kn = synth.bf16(synth.normal((B, Hkv, D), 1000 + i, std=0.5))
        vn = synth.bf16(synth.normal((B, Hkv, D), 5000 + i))
        sr = (torch.randint(0, 6, (B, Hkv), generator=g).float() * 0.5)
        if i % 17 == 0:
            sr[0, 0] = float("nan")
        kv.cache_step(st["kc"], st["vc"], st["slot_pos"], st["slot_score"], kn.cuda(), vn.cuda(),
                      q, s, w, delay, scores_r=sr.cuda())
        oracle.cache_step(ost, bits(kn), bits(vn), sr.numpy(), s, w, delay, q)
    torch.cuda.synchronize()
    _same_state(st, ost, "after steps")


def test_cache_step_mlp_matches_score_kernel(kv):
    """The in-step scorer gives the same bits as kvpop_score_mlp on the same
    key, and both agree with the oracle MLP within tolerance."""
    B, Hkv, D, hidden, s, w, k = 2, 4, 128, 64, 4, 32, 64
    budget = s + w + k
    S0, delay = 300, 7
    st = _prefix_state(kv, B, Hkv, S0, D, s, w, budget, seed=3)
    w1, b1, w2, b2 = [t.cuda() for t in synth.mlp_weights(Hkv, D, hidden, seed=9)]
    keys = []
    for i in range(40):
        q = S0 + i
        kn = synth.bf16(synth.normal((B, Hkv, D), 700 + i, std=0.5)).cuda()
        vn = synth.bf16(synth.normal((B, Hkv, D), 900 + i)).cuda()
        keys.append(kn)
        kv.cache_step(st["kc"], st["vc"], st["slot_pos"], st["slot_score"], kn, vn, q, s, w,
                      delay, mlp=(w1, b1, w2, b2))
        r = q - delay
        if r >= S0:
            slot = s + k + (r % w)
            kr = keys[r - S0][:, :, None, :].contiguous()
            ref = kv.score_mlp(kr, w1, b1, w2, b2)[:, :, 0]
            got = st["slot_score"][:, :, slot]
            assert torch.equal(got.view(torch.int32), ref.view(torch.int32)), i
            o = oracle.mlp_score(f32(kr), *(t.cpu().numpy() for t in (w1, b1, w2, b2)))[:, :, 0]
            assert_close(f32(got), o, MLP_ATOL, MLP_RTOL, "mlp in step")


def _decode_state(B, Hkv, D, s, w, budget, seed):
    """A full bounded cache as the prefix selection leaves it."""
    S0 = 4 * budget
    k = synth.bf16(synth.normal((B, Hkv, S0, D), seed, std=0.5)).cuda()
    v = synth.bf16(synth.normal((B, Hkv, S0, D), seed + 1)).cuda()
    sc = synth.scores((B, Hkv, S0), seed + 2, kind="normal").cuda()
    sp, ss, kc, vc = kv_lib().evict_select(sc, s, w, budget, k, v)
    return S0, {"kc": kc, "vc": vc, "sp": sp, "ss": ss}


def kv_lib():
    return ensure_built()


@pytest.mark.parametrize("B,Hq,Hkv,D,k_sel,use_mlp", [
    (64, 32, 8, 128, 60, True), (64, 32, 8, 128, 60, False), (2, 8, 2, 64, 60, True),
    (3, 4, 4, 128, 60, False),
    (1, 8, 2, 128, 1000, True)])  # few rows, long budget: slots split, two launches
def test_decode_step_matches_two_calls(kv, B, Hq, Hkv, D, k_sel, use_mlp):
    """kvpop_decode_step (one launch when every (b, KV head) row has its own
    workgroup, else the two kernels) leaves the same cache state, bit for
    bit, and gives the same o and lse as kvpop_cache_step followed by
    kvpop_decode_attend."""
    s, w, delay, hidden = 4, 32, 5, 64
    budget = s + w + k_sel
    S0, a = _decode_state(B, Hkv, D, s, w, budget, seed=B + D)
    b = {n: t.clone() for n, t in a.items()}
    mlp = [t.cuda() for t in synth.mlp_weights(Hkv, D, hidden, seed=8)] if use_mlp else None
    g = torch.Generator().manual_seed(11)
    for i in range(40):
        q = S0 + i
        kn = synth.bf16(synth.normal((B, Hkv, D), 300 + i, std=0.5)).cuda()
        vn = synth.bf16(synth.normal((B, Hkv, D), 600 + i)).cuda()
        qv = synth.bf16(synth.normal((B, Hq, D), 900 + i, std=0.5)).cuda()
        sr = None if use_mlp else (torch.randint(0, 6, (B, Hkv), generator=g).float() * 0.5).cuda()
        kv.cache_step(a["kc"], a["vc"], a["sp"], a["ss"], kn, vn, q, s, w, delay, mlp=mlp, scores_r=sr)
        oa, la = kv.decode_attend(qv, a["kc"], a["vc"], a["sp"])
        ob, lb = kv.decode_step(qv, b["kc"], b["vc"], b["sp"], b["ss"], kn, vn, q, s, w, delay,
                                mlp=mlp, scores_r=sr)
        torch.cuda.synchronize()
        for n in ("sp", "ss", "kc", "vc"):
            x, y = a[n], b[n]
            if x.dtype != torch.int32:
                x, y = x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32), \
                    y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32)
            assert torch.equal(x, y), (i, n)
        assert torch.equal(oa.view(torch.int32), ob.view(torch.int32)), i
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), i
