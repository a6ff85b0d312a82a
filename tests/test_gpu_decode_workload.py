"""GPU parity of the one-launch decode steps at the bounded-decode workload's
shape, against the CPU oracle, through the C ABI.

Shape: 64 sequences, 32 query / 8 KV heads, D = 128, budget 4096 per KV head
(4 sinks + 256-token window + 3836 kept long-range tokens), delay 16.  With
512 (b, KV head) rows the device is full, so kvpop_decode_step and
kvpop_decode_step_mlstm run the scorer, the cache step and the attention of
a row in one workgroup (one launch per step): the code path behind both
decode throughput figures of the bench.

KVpop summary (arXiv 2607.05061v2, paperlayer.ai): Sec. 3 (fixed-budget
pruning; a token is scored while in the window and judged when it leaves
it), App. C.1 (decoding over the retained entries; B = s + w + k), App. E.2
(headwise MLP scorer), App. E.3-E.4 (delayed mLSTM scorer; the newly
eligible token is u = q - w).

Method of the check: the prefix is retained by kvpop_evict_select; eight
sampled (b, KV head) rows are rebuilt on the host by the oracle's selection
and compaction from the same fp32 prefix scores, then replayed step by step
with the oracle's cache step, fed the scores the GPU scorer produced (read
back from the slot scores).  After every step the GPU rows must equal the
oracle's state bit for bit (slot positions, slot scores, K and V caches);
o and lse of the row's query heads are compared with the oracle's decode
attention over its own state; the GPU scores with the oracle's scorers.
Tolerances: o |d| <= 1e-5 + 2e-3 |ref| (fp32 output; + 2^-8 |ref| for bf16),
lse |d| <= 1e-4, scores |d| <= 1e-5 + 1e-4 |ref|.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import MLP_ATOL, MLP_RTOL, O_ATOL, O_RTOL, assert_close, bits, ensure_built, f32

pytestmark = pytest.mark.gpu

W = synth.DECODE
S0 = 6144          # prefix length: 5884 eligible tokens, 3836 of them kept
N_STEPS = 20
ROWS = ((0, 0), (7, 3), (13, 7), (22, 1), (31, 5), (40, 2), (51, 6), (63, 4))
BI = np.array([r[0] for r in ROWS])
HI = np.array([r[1] for r in ROWS])
P_FEAT, E_VAL = 32, 64


@pytest.fixture(scope="module")
def kv():
    return ensure_built()


def _rows(t):
    """The sampled (b, KV head) rows of a [B, Hkv, ...] device tensor, on the host."""
    return t[torch.as_tensor(BI, device=t.device), torch.as_tensor(HI, device=t.device)].cpu()


def _prefix(kv, scores):
    """Retain the prefix on the GPU; rebuild the sampled rows with the oracle."""
    dev = "cuda"
    kp = synth.bf16(synth.normal((W.B, W.Hkv, S0, W.D), 31, dev, W.std))
    vp = synth.bf16(synth.normal((W.B, W.Hkv, S0, W.D), 32, dev, W.std))
    sc = scores(kp)
    sp, ss, kc, vc = kv.evict_select(sc, W.n_sink, W.window, W.budget, kp, vp)
    torch.cuda.synchronize()
    osp, oss = oracle.select(_rows(sc).numpy()[:, None], W.n_sink, W.window, W.budget)
    ost = {"slot_pos": osp, "slot_score": oss,
           "kc": oracle.gather(bits(_rows(kp))[:, None], osp),
           "vc": oracle.gather(bits(_rows(vp))[:, None], osp)}
    gpu = {"slot_pos": sp, "slot_score": ss, "kc": kc, "vc": vc}
    _same(gpu, ost, "prefix")
    return kp, vp, sc, gpu, ost


def _same(gpu, ost, what):
    assert np.array_equal(_rows(gpu["slot_pos"]).numpy(), ost["slot_pos"][:, 0]), f"{what}: slot_pos"
    gs = _rows(gpu["slot_score"]).numpy().view(np.uint32)
    assert np.array_equal(gs, ost["slot_score"][:, 0].view(np.uint32)), f"{what}: slot_score"
    assert np.array_equal(bits(_rows(gpu["kc"])), ost["kc"][:, 0]), f"{what}: k cache"
    assert np.array_equal(bits(_rows(gpu["vc"])), ost["vc"][:, 0]), f"{what}: v cache"


def _new_token(i):
    dev = "cuda"
    kn = synth.bf16(synth.normal((W.B, W.Hkv, W.D), 100 + i, dev, W.std))
    vn = synth.bf16(synth.normal((W.B, W.Hkv, W.D), 300 + i, dev, W.std))
    qn = synth.bf16(synth.normal((W.B, W.Hq, W.D), 500 + i, dev, W.std))
    return kn, vn, qn


def _check_attention(o, lse, qn, ost, bf16_out, what):
    """o, lse of every query head of the sampled rows against the oracle's
    decode attention over the oracle's own (replayed) state."""
    G = W.Hq // W.Hkv
    qv = qn.view(W.B, W.Hkv, G, W.D)
    qr = f32(_rows(qv))                                     # [8, G, D]
    kcf = oracle.bf16_bits_to_f32(ost["kc"])                # [8, 1, budget, D]
    vcf = oracle.bf16_bits_to_f32(ost["vc"])
    oo, ol = oracle.decode_attend(qr, kcf, vcf, ost["slot_pos"])
    og = f32(_rows(o.view(W.B, W.Hkv, G, W.D)))
    lg = f32(_rows(lse.view(W.B, W.Hkv, G)))
    assert_close(og, oo, O_ATOL, O_RTOL + (2.0 ** -8 if bf16_out else 0.0), f"{what}: o")
    assert_close(lg, ol, 1e-4, 0.0, f"{what}: lse")


def test_decode_step_mlp_at_workload_shape(kv):
    """kvpop_decode_step with the in-step MLP scorer (hidden 64, delay 16)."""
    s, w, delay, hidden = W.n_sink, W.window, W.extra["delay"], W.extra["hidden"]
    kk = W.budget - s - w
    mlp = [t.cuda() for t in synth.mlp_weights(W.Hkv, W.D, hidden, seed=33)]
    kp, vp, sc, gpu, ost = _prefix(kv, lambda kp: kv.score_mlp(kp, *mlp))
    # the prefix scores themselves against the oracle's MLP (sampled tokens)
    toks = np.unique(np.concatenate([[0, s, S0 - w - 1, S0 - 1], np.arange(7, S0, 389)]))
    w_np = [t.cpu().numpy() for t in mlp]
    for j, (b, h) in enumerate(ROWS):
        ref = oracle.mlp_score(f32(kp[b, h, toks])[None, None], w_np[0][h:h + 1], w_np[1][h:h + 1],
                               w_np[2][h:h + 1], w_np[3][h:h + 1])[0, 0]
        assert_close(f32(sc[b, h, toks]), ref, MLP_ATOL, MLP_RTOL, f"prefix score row {j}")
    dws = torch.empty(max(kv.workspace_bytes(kv.OP_DECODE, kv.dims(W.B, W.Hq, W.Hkv, W.budget, W.D)),
                          16), dtype=torch.uint8, device="cuda")
    kept = dropped = 0
    for i in range(N_STEPS):
        pos = S0 + i
        kn, vn, qn = _new_token(i)
        bf16_out = i == N_STEPS - 1
        pre = ost["slot_pos"].copy()
        print(f"mlp decode step {i} pos {pos}", flush=True)
        o, lse = kv.decode_step(qn, gpu["kc"], gpu["vc"], gpu["slot_pos"], gpu["slot_score"], kn, vn,
                                pos, s, w, delay, mlp=mlp,
                                out_dtype=torch.bfloat16 if bf16_out else torch.float32,
                                workspace=dws)
        torch.cuda.synchronize()
        r = pos - delay
        ring_r = s + kk + r % w
        sr = _rows(gpu["slot_score"])[:, ring_r].numpy().astype(np.float32)
        oracle.cache_step(ost, bits(_rows(kn))[:, None], bits(_rows(vn))[:, None], sr[:, None],
                          s, w, delay, pos)
        _same(gpu, ost, f"step {i}")
        # the GPU's delayed score of r against the oracle's MLP on r's cached key
        kr = oracle.bf16_bits_to_f32(ost["kc"][:, 0, ring_r])
        for j, (b, h) in enumerate(ROWS):
            ref = oracle.mlp_score(kr[j][None, None, None], w_np[0][h:h + 1], w_np[1][h:h + 1],
                                   w_np[2][h:h + 1], w_np[3][h:h + 1])[0, 0]
            assert_close(sr[j:j + 1], ref, MLP_ATOL, MLP_RTOL, f"step {i} row {j} delayed score")
        u = pos - w
        now = ost["slot_pos"][:, 0, s:s + kk]
        got_in = (now == u).any(axis=1)
        kept += int(got_in.sum())
        dropped += int((~got_in).sum())
        assert not (pre[:, 0, s:s + kk] == u).any()
        _check_attention(o, lse, qn, ost, bf16_out, f"step {i}")
    # both outcomes of the exit decision were exercised
    assert kept > 0 and dropped > 0, (kept, dropped)


def _mlstm_params(H, D, seed):
    g = torch.Generator().manual_seed(seed)
    X = 2 * D
    r = lambda *sh: torch.randn(sh, generator=g, dtype=torch.float32)
    return {"wk": r(H, P_FEAT, X) / X ** 0.5, "wr": r(H, P_FEAT, X) / X ** 0.5,
            "wv": r(H, E_VAL, X) / X ** 0.5, "wi": r(H, X) / X ** 0.5, "bi": torch.zeros(H),
            "wf": r(H, X) / X ** 0.5, "bf": torch.full((H,), 3.0), "wo": r(H, E_VAL) / 8.0,
            "bo": torch.zeros(H)}


def _worst_kept(ss, sp):
    """Score of the worst kept token of a pool: lowest score, among equal
    scores the highest position (the pools here hold no NaN)."""
    order = np.lexsort((-sp.astype(np.int64), ss))
    return ss[order[0]]


def test_decode_step_mlstm_at_workload_shape(kv):
    """kvpop_decode_step_mlstm: the scorer state takes the new token and reads
    out the exiting one, which the cache step keeps or drops at once.

    The exiting token's GPU score is read back where it was kept; a dropped
    token leaves no score behind, so the oracle's cache step is then handed a
    NaN (which never displaces a kept token) and the oracle's own mLSTM score
    of that token must not rank above the worst kept one beyond the score
    tolerance.  Prefix scores are N(0, 0.04^2), the spread of the random-init
    scorer's outputs, so both outcomes occur."""
    s, w = W.n_sink, W.window
    kk = W.budget - s - w
    dev = "cuda"
    kp, vp, sc, gpu, ost = _prefix(kv, lambda kp: synth.normal((W.B, W.Hkv, S0), 34, dev, 0.04))
    pr = _mlstm_params(W.Hkv, W.D, seed=35)
    prd = {a: t.cuda() for a, t in pr.items()}
    state = kv.mlstm_state(W.B, W.Hkv)
    # the last w prefix tokens enter the scorer state first (no read-out)
    for t in range(S0 - w, S0):
        kv.mlstm_step(kp[:, :, t].contiguous(), vp[:, :, t].contiguous(), prd, state, t, s, w)
    # the oracle's scan over the same token sequence: positions S0-w .. S0+N-1
    toks_k = [f32(_rows(kp[:, :, S0 - w:S0]))]
    toks_v = [f32(_rows(vp[:, :, S0 - w:S0]))]
    news = [_new_token(i) for i in range(N_STEPS)]
    toks_k += [f32(_rows(kn))[:, None] for kn, _, _ in news]
    toks_v += [f32(_rows(vn))[:, None] for _, vn, _ in news]
    seq_k = np.concatenate(toks_k, axis=1)[:, None]       # [8, 1, w + N, D]
    seq_v = np.concatenate(toks_v, axis=1)[:, None]
    ref_sc = np.empty((len(ROWS), N_STEPS))
    ref_state = []
    for j, (b, h) in enumerate(ROWS):
        ph = {a: t[h:h + 1].numpy() for a, t in pr.items()}
        scj, stj = oracle.mlstm_scores(seq_k[j:j + 1], seq_v[j:j + 1], ph, w, want_state=True)
        ref_sc[j] = scj[0, 0, :N_STEPS]                     # u = S0 - w + i, read out at S0 + i
        ref_state.append(stj)
    dws = torch.empty(max(kv.workspace_bytes(kv.OP_DECODE, kv.dims(W.B, W.Hq, W.Hkv, W.budget, W.D)),
                          16), dtype=torch.uint8, device=dev)
    kept = dropped = 0
    for i, (kn, vn, qn) in enumerate(news):
        pos = S0 + i
        u = pos - w
        ring_u = s + kk + u % w
        worst = [_worst_kept(ost["slot_score"][j, 0, s:s + kk], ost["slot_pos"][j, 0, s:s + kk])
                 for j in range(len(ROWS))]
        print(f"mlstm decode step {i} pos {pos}", flush=True)
        o, lse = kv.decode_step_mlstm(qn, gpu["kc"], gpu["vc"], gpu["slot_pos"], gpu["slot_score"],
                                      kn, vn, prd, state, pos, s, w, workspace=dws)
        torch.cuda.synchronize()
        gsp = _rows(gpu["slot_pos"]).numpy()
        gss = _rows(gpu["slot_score"]).numpy()
        for j in range(len(ROWS)):
            hit = np.nonzero(gsp[j, s:s + kk] == u)[0]
            ref = ref_sc[j, i]
            if hit.size:
                kept += 1
                sg = gss[j, s + hit[0]]
                assert_close(np.array([sg]), np.array([ref]), MLP_ATOL, MLP_RTOL,
                             f"step {i} row {j} mlstm score")
                ost["slot_score"][j, 0, ring_u] = sg
            else:
                dropped += 1
                assert ref <= worst[j] + MLP_ATOL + MLP_RTOL * abs(worst[j]), \
                    f"step {i} row {j}: dropped, yet its oracle score {ref} ranks above {worst[j]}"
                ost["slot_score"][j, 0, ring_u] = np.float32(np.nan)
        nan_r = np.full((len(ROWS), 1), np.nan, np.float32)
        oracle.cache_step(ost, bits(_rows(kn))[:, None], bits(_rows(vn))[:, None], nan_r, s, w, 0, pos)
        _same(gpu, ost, f"step {i}")
        _check_attention(o, lse, qn, ost, False, f"step {i}")
    assert kept > 0 and dropped > 0, (kept, dropped)
    # the scorer state after all steps against the oracle's scan
    st = _rows(state).numpy()
    F = 2 * P_FEAT
    for j in range(len(ROWS)):
        C, nr, m = (x[0, 0] for x in ref_state[j])
        Cg = st[j, :E_VAL * F].reshape(E_VAL, F)
        assert (np.abs(Cg - C) <= 1e-5 * np.abs(C).max() + 1e-4 * np.abs(C)).all(), f"row {j}: C"
        ng = st[j, E_VAL * F:E_VAL * F + F]
        assert (np.abs(ng - nr) <= 1e-5 * np.abs(nr).max() + 1e-4 * np.abs(nr)).all(), f"row {j}: n"
        np.testing.assert_allclose(st[j, E_VAL * F + F], m, rtol=1e-5, atol=1e-5)
