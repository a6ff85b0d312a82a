"""Benchmark of the KVpop hot path on one MI355X.

Timed step (the headline): one pass of the whole hot path over the
Qwen3-8B-shaped 36-layer prefill (B=1, 32 query / 8 KV heads, D=128,
S=32768, RoPE, w=256, s=4, budget 8192 per KV head), on every layer's own
resident inputs: causal LSE pass -> transposed future-attention target (SUM
over the group) -> retention + compaction of K/V to the budget -> one
bounded-cache decode step over the fresh cache (delayed MLP scoring, then
decode attention).  value = 36 * B * Hkv * S KV-head keys scored per second
of step time.  roofline: the transposed pass (kvpop_future_attn_target),
the dominant call, against the dense bf16 MFMA peak.

Also reported, each under its own key: the same step on the Qwen3-4B layer,
the target variants, retention and the sparse normalizer on that layer, the
skewed 16k batch, the attention-output mode of the main pass, the sparse
normalizer on one 32k layer, the bounded-cache decode workload (64
sequences, 36 layers, budget 4096, 512 steps; steps/s with its HBM
roofline) and the CPU oracle timed on bounded samples.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]   (defaults: K=5, W=2)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

import synth  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
FP32_VECTOR_PEAK_TFS = 157.3     # MI355X fp32 vector (counts packed FMA; one FMA per lane per cycle is half)

# HBM bytes of one kvpop_future_attn_target call (transposed pass + merge) on
# one layer of the 36-layer prefill, from two rocprofv3 --pmc runs (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch) each scaled by what the same counter
# reads for a torch copy of known size (`bench.py --calibrate-copy`).  Valid
# only for the kernel code it was taken on (sources_digest): bench reports
# null once that changes.
TRAFFIC_SOURCES = ("future_target.hip", "common.h", "launch.h")
TRAFFIC = {"sha256": "ea2334b72027295d40a618d36fbedd75f07b2ac8d2ca5c0c104302f44d1dc79d",
           "fetch_bytes": 2 * (446061.5 + 4319.0) * 1024, "write_bytes": (8576.0 + 1024.0) * 1024}
# HBM bytes per dispatch of the HBM-bound kernels the bench reports, from the
# same pair of counter runs with the same scaling (FETCH_SIZE x 2, WRITE_SIZE
# x 1), each valid only for the sources it was taken on.
COUNTERS = {
    "decode_step": {"sources": ("decode_step.hip", "decode_dev.h", "cache_step_dev.h", "mlstm_dev.h",
                                "common.h", "launch.h"),
                    "fetch_kib": 532937.5, "write_kib": 824.3,
                    "per": "decode_step_kernel<128, 4> launch: one layer-step of 64 sequences x 8 KV "
                           "heads over budget 4096"},
    "select_gather_prefill": {"sources": ("select.hip", "common.h", "launch.h"),
                              "fetch_kib": 20619.6, "write_kib": 33281.6,
                              "per": "select_kernel<32, true, true> launch: 8 rows of 32768 scores, "
                                     "budget 8192, selection and compaction of K and V (32 "
                                     "workgroups per row)"},
    "select_decode_prefix": {"sources": ("select.hip", "common.h", "launch.h"),
                             "fetch_kib": 32919.4, "write_kib": 16416.0,
                             "per": "select_kernel<32, true, false> launch: 512 rows of 32768 scores, "
                                    "budget 4096"},
    "gather_decode_prefix": {"sources": ("select.hip", "common.h", "launch.h"),
                             "fetch_kib": 532515.1, "write_kib": 1048649.4,
                             "per": "gather_kernel launch: 512 rows x 4096 slots of K and V"},
}
COUNTER_SHA = {"decode": "e13a93995337dc717550ad10a07325b82b8cdc39af6460c184f22176236abdfc",
               "select": "5ce051bb1a59368f64d107b40b90e5b731dc660263b2d45f59f60d506ae08149"}
METRIC = "future-attn target keys/s + MFMA util; bounded-cache decode steps/s + HBM util"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def target_flops(w):
    """Algorithmic flops of the two attention passes (QK^T only, masked pairs
    excluded): causal pass 2*D*S(S+1)/2*Hq*B; transposed pass
    2*D*(S-w)(S-w+1)/2*Hq*B."""
    f_fwd = 2.0 * w.D * w.S * (w.S + 1) / 2 * w.Hq * w.B
    n = max(w.S - w.window, 0)
    f_tr = 2.0 * w.D * n * (n + 1) / 2 * w.Hq * w.B
    return f_fwd, f_tr


class TargetStep:
    """Buffers and one step of the hot path on the layer workload."""

    def __init__(self, kv, w, seed=7, hidden=64, delay=16):
        dev = torch.device("cuda")
        self.kv, self.w, self.delay = kv, w, delay
        self.q, self.k, self.v = synth.attention_inputs(w, seed=seed, device=dev)
        self.lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
        self.mass = torch.empty((w.B, w.Hkv, w.S), dtype=torch.float32, device=dev)
        d = kv.dims(w.B, w.Hq, w.Hkv, w.S, w.D)
        self.ws = torch.empty(kv.workspace_bytes(kv.OP_FUTURE_TARGET, d, w.window), dtype=torch.uint8,
                              device=dev)
        self.fws = torch.empty(max(kv.workspace_bytes(kv.OP_FWD_LSE, d), 16), dtype=torch.uint8,
                               device=dev)
        self.sp = torch.empty((w.B, w.Hkv, w.budget), dtype=torch.int32, device=dev)
        self.ss = torch.empty((w.B, w.Hkv, w.budget), dtype=torch.float32, device=dev)
        self.kc = torch.empty((w.B, w.Hkv, w.budget, w.D), dtype=torch.bfloat16, device=dev)
        self.vc = torch.empty_like(self.kc)
        self.mlp = [t.to(dev) for t in synth.mlp_weights(w.Hkv, w.D, hidden, seed=seed)]
        self.k_new = synth.bf16(synth.normal((w.B, w.Hkv, w.D), seed + 11, dev, w.std))
        self.v_new = synth.bf16(synth.normal((w.B, w.Hkv, w.D), seed + 12, dev, w.std))
        self.q_new = synth.bf16(synth.normal((w.B, w.Hq, w.D), seed + 13, dev, w.std))
        self.o = torch.empty((w.B, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
        dd = kv.dims(w.B, w.Hq, w.Hkv, w.budget, w.D)
        nb = kv.workspace_bytes(kv.OP_DECODE, dd)
        self.dws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)

    def run(self, ev=None, ev_target=None):
        """One step.  ev: four events around the passes (instrumented
        breakdown); ev_target: two events around the target call only."""
        kv, w = self.kv, self.w
        if ev:
            ev[0].record()
        kv.fwd_lse(self.q, self.k, out=self.lse, workspace=self.fws)
        if ev:
            ev[1].record()
        if ev_target:
            ev_target[0].record()
        kv.future_attn_target(self.q, self.k, self.lse, w.window, agg="sum", out=self.mass,
                              workspace=self.ws)
        if ev_target:
            ev_target[1].record()
        if ev:
            ev[2].record()
        kv.evict_select(self.mass, w.n_sink, w.window, w.budget, self.k, self.v, out_pos=self.sp,
                        out_score=self.ss, out_k=self.kc, out_v=self.vc)
        kv.cache_step(self.kc, self.vc, self.sp, self.ss, self.k_new, self.v_new, w.S, w.n_sink,
                      w.window, self.delay, mlp=self.mlp)
        kv.decode_attend(self.q_new, self.kc, self.vc, self.sp, out_dtype=torch.bfloat16,
                         want_lse=False, out=self.o, workspace=self.dws)
        if ev:
            ev[3].record()


def bench_target(kv, steps, warmup):
    """Timed region: `steps` steps between two events, with one more pair of
    events around each step's target call (the dominant kernel; two events
    per step cost ~1.5% of the step, four ~6%).  After it, the same number
    of steps with events around every pass gives the per-pass breakdown."""
    w = synth.QWEN4B
    st = TargetStep(kv, w)
    for _ in range(warmup):
        st.run()
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)
    evt = [[E(), E()] for _ in range(steps)]
    t0, t1 = E(), E()
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        st.run(ev_target=evt[i])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    t_tr = sum(e[0].elapsed_time(e[1]) for e in evt) / steps
    # instrumented breakdown (not the timed region)
    evs = [[E() for _ in range(4)] for _ in range(steps)]
    a, b = E(), E()
    a.record()
    for i in range(steps):
        st.run(evs[i])
    b.record()
    torch.cuda.synchronize()
    brk = {"ms_per_step": a.elapsed_time(b) / steps,
           "fwd_lse": sum(e[0].elapsed_time(e[1]) for e in evs) / steps,
           "future_attn_target": sum(e[1].elapsed_time(e[2]) for e in evs) / steps,
           "select_gather_decode": sum(e[2].elapsed_time(e[3]) for e in evs) / steps}
    f_fwd, f_tr = target_flops(w)
    return st, ms, t_tr, brk, f_fwd, f_tr


class PrefillStep:
    """Buffers and one step of the hot path over every layer of a
    multi-layer prefill workload (the layers' inputs resident in HBM)."""

    def __init__(self, kv, w, seed_base=4000, hidden=64, delay=16):
        dev = torch.device("cuda")
        self.kv, self.w, self.delay = kv, w, delay
        log(f"{w.name}: generating {w.layers} layers of inputs")
        self.ins = [synth.attention_inputs(w, seed=seed_base + l, device=dev) for l in range(w.layers)]
        d = kv.dims(w.B, w.Hq, w.Hkv, w.S, w.D)
        self.lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
        self.mass = torch.empty((w.B, w.Hkv, w.S), dtype=torch.float32, device=dev)
        self.tws = torch.empty(kv.workspace_bytes(kv.OP_FUTURE_TARGET, d, w.window),
                               dtype=torch.uint8, device=dev)
        self.fws = torch.empty(max(kv.workspace_bytes(kv.OP_FWD_LSE, d), 16), dtype=torch.uint8,
                               device=dev)
        self.sp = torch.empty((w.B, w.Hkv, w.budget), dtype=torch.int32, device=dev)
        self.ss = torch.empty((w.B, w.Hkv, w.budget), dtype=torch.float32, device=dev)
        self.kc = torch.empty((w.B, w.Hkv, w.budget, w.D), dtype=torch.bfloat16, device=dev)
        self.vc = torch.empty_like(self.kc)
        self.mlps = [[t.to(dev) for t in synth.mlp_weights(w.Hkv, w.D, hidden, seed=seed_base + l)]
                     for l in range(w.layers)]
        self.k_new = synth.bf16(synth.normal((w.B, w.Hkv, w.D), seed_base + 101, dev, w.std))
        self.v_new = synth.bf16(synth.normal((w.B, w.Hkv, w.D), seed_base + 102, dev, w.std))
        self.q_new = synth.bf16(synth.normal((w.B, w.Hq, w.D), seed_base + 103, dev, w.std))
        self.o = torch.empty((w.B, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
        dd = kv.dims(w.B, w.Hq, w.Hkv, w.budget, w.D)
        self.dws = torch.empty(max(kv.workspace_bytes(kv.OP_DECODE, dd), 16), dtype=torch.uint8,
                               device=dev)

    def layer(self, i, ev=None):
        """One layer of the step; ev: five events around its four passes."""
        kv, w = self.kv, self.w
        q, k, v = self.ins[i]
        if ev:
            ev[0].record()
        kv.fwd_lse(q, k, out=self.lse, workspace=self.fws)
        if ev:
            ev[1].record()
        kv.future_attn_target(q, k, self.lse, w.window, agg="sum", out=self.mass, workspace=self.tws)
        if ev:
            ev[2].record()
        kv.evict_select(self.mass, w.n_sink, w.window, w.budget, k, v, out_pos=self.sp,
                        out_score=self.ss, out_k=self.kc, out_v=self.vc)
        if ev:
            ev[3].record()
        kv.decode_step(self.q_new, self.kc, self.vc, self.sp, self.ss, self.k_new, self.v_new, w.S,
                       w.n_sink, w.window, self.delay, mlp=self.mlps[i], out_dtype=torch.bfloat16,
                       want_lse=False, out=self.o, workspace=self.dws)
        if ev:
            ev[4].record()

    def run(self, evs=None):
        for i in range(self.w.layers):
            self.layer(i, evs[i] if evs else None)


def bench_prefill_step(kv, w, steps, warmup):
    """The headline: `steps` timed steps (after `warmup`) of PrefillStep,
    between two events; events around every pass of every layer give the
    per-pass means (at ~7.4 ms per layer their cost is negligible).  The
    roofline of the transposed pass is its flops per call over the mean of
    its calls' event durations in the timed steps."""
    st = PrefillStep(kv, w)
    for i in range(warmup):
        st.run()
        log(f"{w.name}: warm-up step {i + 1}/{warmup} issued")
    torch.cuda.synchronize()
    E = lambda: torch.cuda.Event(enable_timing=True)
    evs = [[[E() for _ in range(5)] for _ in range(w.layers)] for _ in range(steps)]
    a, b = E(), E()
    a.record()
    for i in range(steps):
        st.run(evs[i])
        log(f"{w.name}: timed step {i + 1}/{steps} issued")
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    n = steps * w.layers
    flat = [e for step in evs for e in step]
    per = [sum(e[j].elapsed_time(e[j + 1]) for e in flat) / n for j in range(4)]
    t_fwd, t_tr, t_sel, t_dec = per
    f_fwd, f_tr = target_flops(w)
    rows = w.B * w.Hkv
    sg_bytes = rows * (4 * w.S + 8 * w.budget) + rows * 2 * (2 * w.budget * w.D * 2)
    tf = lambda f, ms_: f / (ms_ / 1e3) / 1e12
    out = {"ms_per_step": ms, "keys_per_s": w.layers * w.B * w.Hkv * w.S / (ms / 1e3),
           "t_target_ms": t_tr, "f_target": f_tr,
           "per_layer_ms": {"fwd_lse": t_fwd, "future_attn_target": t_tr, "select_gather": t_sel,
                            "decode_step": t_dec},
           "fwd_lse": {"flops": f_fwd, "tflops": tf(f_fwd, t_fwd),
                       "frac": tf(f_fwd, t_fwd) / MFMA_BF16_PEAK_TFLOPS},
           "future_attn_target": {"flops": f_tr, "tflops": tf(f_tr, t_tr),
                                  "frac": tf(f_tr, t_tr) / MFMA_BF16_PEAK_TFLOPS},
           "select_gather": {"bytes": sg_bytes, "achieved": sg_bytes / (t_sel / 1e3) / 1e9,
                             "unit": "GB/s",
                             "frac": sg_bytes / (t_sel / 1e3) / 1e9 / HBM_PEAK_GBS,
                             "counters": _one_counter("select_gather_prefill", t_sel),
                             "note": "8 rows: bound by the latency of a row's selection"},
           "decode_step": {"ms": t_dec, "sequences": w.B, "slots": w.budget,
                           "entry_point": "kvpop_decode_step"}}
    del st
    torch.cuda.empty_cache()
    return out


def target_flops_lookahead(w, lookahead):
    """Algorithmic flops of the transposed pass with a finite lookahead L:
    key t counts queries t+w .. min(S-1, t+w+L), so 2*D*sum_j min(L+1, j)
    over j = 1..S-w, per query head."""
    n = max(w.S - w.window, 0)
    m = lookahead + 1
    pairs = n * (n + 1) // 2 if m >= n else m * (m + 1) // 2 + (n - m) * m
    return 2.0 * w.D * pairs * w.Hq * w.B


def bench_target_variants(kv, st, reps=20):
    """The pages' other target forms on the same layer inputs: MAX over the
    group (App. B.1, per-query-head sums kept), and a finite lookahead with
    count normalisation (App. B.2)."""
    w = st.w
    variants = {
        "max_per_qhead": (dict(agg="max", per_qhead=True), target_flops(w)[1]),
        "sum_lookahead512_count_normalized": (dict(agg="sum", lookahead=512, count_normalize=True),
                                              target_flops_lookahead(w, 512)),
    }
    out = {}
    for name, (kw, flops) in variants.items():
        def call():
            kv.future_attn_target(st.q, st.k, st.lse, w.window, out=st.mass, workspace=st.ws, **kw)
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            call()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        tf = flops / (ms / 1e3) / 1e12
        out[name] = {"ms": ms, "flops": flops, "tflops": tf, "frac": tf / MFMA_BF16_PEAK_TFLOPS}
    return out


def bench_retention(kv, st, reps=50):
    """Selection alone and selection + compaction on the layer's fp32 mass,
    with their algorithmic HBM bytes: select reads the scores of every row
    and writes slot positions and scores (4 S + 8 budget bytes per row);
    the gather reads and writes every kept K and V row (4 budget D bytes per
    row each way)."""
    w = st.w
    rows = w.B * w.Hkv
    sel_bytes = rows * (4 * w.S + 8 * w.budget)
    gat_bytes = rows * 2 * (2 * w.budget * w.D * 2)

    def t_ms(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_sel = t_ms(lambda: kv.evict_select(st.mass, w.n_sink, w.window, w.budget, out_pos=st.sp,
                                         out_score=st.ss))
    t_both = t_ms(lambda: kv.evict_select(st.mass, w.n_sink, w.window, w.budget, st.k, st.v,
                                          out_pos=st.sp, out_score=st.ss, out_k=st.kc, out_v=st.vc))
    gbs = lambda by, ms: by / (ms / 1e3) / 1e9
    return {"rows": rows,
            "select": {"ms": t_sel, "bytes": sel_bytes, "achieved": gbs(sel_bytes, t_sel),
                       "unit": "GB/s", "frac": gbs(sel_bytes, t_sel) / HBM_PEAK_GBS},
            "select_gather": {"ms": t_both, "bytes": sel_bytes + gat_bytes,
                              "achieved": gbs(sel_bytes + gat_bytes, t_both), "unit": "GB/s",
                              "frac": gbs(sel_bytes + gat_bytes, t_both) / HBM_PEAK_GBS},
            "note": "8 rows of 4096 scores: launch- and latency-bound, not bandwidth-bound"}


def bench_attention_output(kv, w, reps=5, seed=6000):
    """The main pass with its attention output (App. D.4 first step, App. I)
    on one layer of a workload: kvpop_fwd_lse with v and a bf16 o, beside
    the LSE-only call on the same inputs.  Algorithmic flops of the output
    mode: 4 D per causal (query, key) pair -- the score product and the
    P.V product -- i.e. twice those of the LSE-only pass."""
    dev = torch.device("cuda")
    q, k, v = synth.attention_inputs(w, seed=seed, device=dev)
    d = kv.dims(w.B, w.Hq, w.Hkv, w.S, w.D)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    aws = torch.empty(kv.workspace_bytes(kv.OP_FWD_ATTN, d), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(kv.workspace_bytes(kv.OP_FWD_LSE, d), 16), dtype=torch.uint8, device=dev)

    def t_ms(fn):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_out = t_ms(lambda: kv.fwd_lse(q, k, v=v, out=lse, out_o=o, workspace=aws))
    t_lse = t_ms(lambda: kv.fwd_lse(q, k, out=lse, workspace=fws))
    f_lse, _ = target_flops(w)
    tf = lambda f, ms: f / (ms / 1e3) / 1e12
    out = {"workload": w.name, "o_dtype": "bf16", "entry_point": "kvpop_fwd_lse (v, o given)",
           "ms": t_out, "flops": 2 * f_lse, "tflops": tf(2 * f_lse, t_out),
           "frac": tf(2 * f_lse, t_out) / MFMA_BF16_PEAK_TFLOPS,
           "lse_only": {"ms": t_lse, "flops": f_lse, "frac": tf(f_lse, t_lse) / MFMA_BF16_PEAK_TFLOPS},
           "note": "output-mode time includes the V transpose into the workspace"}
    del q, k, v, o, aws
    torch.cuda.empty_cache()
    return out


def live_pairs(until, S):
    """Sum over queries d of |R_d|: key t is retained for d in [t, keep_until[t])."""
    t = torch.arange(S, device=until.device, dtype=torch.int64)
    return int((until.to(torch.int64) - t).clamp_min(0).sum().item())


def listed_flops(until, S, G, D):
    """MFMA flops the listed sparse pass executes: every block of P = 128/G
    queries walks its list, #{t < p0 : keep_until[t] > p0} + (p1 - p0) keys
    rounded up to whole 64-key tiles, for 128 query rows."""
    P = 128 // G
    nb = (S + P - 1) // P
    t = torch.arange(S, device=until.device, dtype=torch.int64)
    u = until.to(torch.int64).reshape(-1, 1, S)
    tiles = 0
    for c0 in range(0, nb, 128):  # blocks in groups, to bound the temporaries
        p0 = torch.arange(c0, min(nb, c0 + 128), device=until.device, dtype=torch.int64) * P
        alive = ((t[None, None, :] < p0[None, :, None]) & (u > p0[None, :, None])).sum(-1)
        n = alive + (torch.clamp(p0 + P, max=S) - p0)[None, :]
        tiles += int(((n + 63) // 64).sum().item())
    return float(tiles) * 2.0 * D * 64 * 128


def bench_sparse(kv, st, reps=20):
    """The target with the sparse normalizer (App. D.3) on the layer inputs:
    the running top-k mask (App. C.1-C.2) over MLP-scorer scores of the
    layer's keys with a per-head decay (lambda_h = 1e-4 * (h + 1)), the
    sparse causal pass, and the transposed pass on its normalizers.  The
    sparse pass runs listed (each block of queries walks the keys retained at
    its first query: about budget + P per block); its algorithmic flops count
    the retained pairs only.  The tested mode (every causal tile read and
    masked) is timed beside it."""
    w = st.w
    dev = st.q.device
    sc = kv.score_mlp(st.k, *st.mlp)
    lam = torch.tensor([1e-4 * (h + 1) for h in range(w.Hkv)], dtype=torch.float32, device=dev)
    until = torch.empty((w.B, w.Hkv, w.S), dtype=torch.int32, device=dev)
    cut = torch.empty_like(until)

    def t_ms(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def mask():
        kv.running_topk(sc, w.n_sink, w.window, w.budget, log_decay=lam, out=until, out_cutoff=cut)

    d = kv.dims(w.B, w.Hq, w.Hkv, w.S, w.D)
    sws = torch.empty(kv.workspace_bytes(kv.OP_FWD_LSE_SPARSE, d, w.budget), dtype=torch.uint8,
                      device=dev)

    def sparse_lse():
        kv.fwd_lse_sparse(st.q, st.k, until, w.budget, out=st.lse, workspace=sws)

    def sparse_lse_tested():
        kv.fwd_lse_sparse(st.q, st.k, until, out=st.lse, workspace=st.fws)

    def target():
        kv.future_attn_target(st.q, st.k, st.lse, w.window, agg="sum", out=st.mass, workspace=st.ws)

    def step():
        mask()
        sparse_lse()
        target()

    t_mask, t_lse, t_tr, t_step = t_ms(mask), t_ms(sparse_lse), t_ms(target), t_ms(step)
    t_tested = t_ms(sparse_lse_tested)
    f_fwd, f_tr = target_flops(w)
    f_live = 2.0 * w.D * w.Hq // w.Hkv * live_pairs(until, w.S)
    f_exec = listed_flops(until, w.S, w.Hq // w.Hkv, w.D)
    tf = lambda f, ms: f / (ms / 1e3) / 1e12
    return {"scores": "kvpop_score_mlp over the layer's keys", "log_decay": "1e-4 * (h + 1)",
            "ms_per_step": t_step, "keys_per_s": w.B * w.Hkv * w.S / (t_step / 1e3),
            "running_topk": {"ms": t_mask},
            "fwd_lse_sparse": {"ms": t_lse, "executed_flops": f_exec,
                               "executed_frac": tf(f_exec, t_lse) / MFMA_BF16_PEAK_TFLOPS,
                               "retained_pair_flops": f_live,
                               "retained_frac": tf(f_live, t_lse) / MFMA_BF16_PEAK_TFLOPS,
                               "mode": "listed", "workspace_bytes": sws.numel(),
                               "tested_mode_ms": t_tested,
                               "tested_mode_frac": tf(f_fwd, t_tested) / MFMA_BF16_PEAK_TFLOPS},
            "future_attn_target": {"ms": t_tr, "tflops": tf(f_tr, t_tr),
                                   "frac": tf(f_tr, t_tr) / MFMA_BF16_PEAK_TFLOPS}}


def bench_sparse_long(kv, w, reps=3):
    """The sparse normalizer on one long-context layer (8 KV heads, the
    workload's budget, seeded scores): the running top-k mask alone, then
    the listed sparse causal pass (key lists + pass), with the dense causal
    pass on the same inputs timed beside it."""
    dev = "cuda"
    q, k, _ = synth.attention_inputs(w, seed=4000, device=dev)
    sc = synth.scores((w.B, w.Hkv, w.S), seed=4000, device=dev)
    until = torch.empty(sc.shape, dtype=torch.int32, device=dev)
    cut = torch.empty_like(until)
    d = kv.dims(w.B, w.Hq, w.Hkv, w.S, w.D)
    sws = torch.empty(kv.workspace_bytes(kv.OP_FWD_LSE_SPARSE, d, w.budget), dtype=torch.uint8,
                      device=dev)
    nb = kv.workspace_bytes(kv.OP_FWD_LSE, d)
    dws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)

    def t_ms(fn):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_mask = t_ms(lambda: kv.running_topk(sc, w.n_sink, w.window, w.budget, out=until,
                                          out_cutoff=cut))
    t_listed = t_ms(lambda: kv.fwd_lse_sparse(q, k, until, w.budget, out=lse, workspace=sws))
    t_dense = t_ms(lambda: kv.fwd_lse(q, k, out=lse, workspace=dws))
    G = w.Hq // w.Hkv
    f_live = 2.0 * w.D * G * live_pairs(until, w.S)
    f_exec = listed_flops(until, w.S, G, w.D)
    f_dense, _ = target_flops(w)
    tf = lambda f, ms: f / (ms / 1e3) / 1e12
    return {"workload": w.name, "rows": w.B * w.Hkv, "seq_len": w.S, "budget": w.budget,
            "running_topk_ms": t_mask,
            "fwd_lse_sparse": {"mode": "listed", "ms": t_listed, "executed_flops": f_exec,
                               "executed_frac": tf(f_exec, t_listed) / MFMA_BF16_PEAK_TFLOPS,
                               "retained_pair_flops": f_live,
                               "retained_frac": tf(f_live, t_listed) / MFMA_BF16_PEAK_TFLOPS,
                               "workspace_bytes": sws.numel()},
            "dense_fwd_lse": {"ms": t_dense, "frac": tf(f_dense, t_dense) / MFMA_BF16_PEAK_TFLOPS}}


def bench_prefill(kv, w, layers=None, reps=1, seed=None, warm=1):
    """The target pipeline on a long-context workload: per layer the causal
    LSE pass, the transposed future-attention pass (SUM over the group) and
    retention + compaction of K/V to the budget, over every layer's own
    resident inputs (generated before the timed region, one seed per layer:
    3000 + l for the skewed workload, 4000 + l for the 36-layer prefill).
    Each pass is timed by its own events; after `warm` untimed warm-up
    layers, `reps` passes over all layers are timed.
    keys/s = layers * B * Hkv * S / (time of one pass over the layers)."""
    dev = torch.device("cuda")
    layers = layers or w.layers
    base = seed if seed is not None else (4000 if w.layers > 1 else 3000)
    ins = [synth.attention_inputs(w, seed=base + l, device=dev) for l in range(layers)]
    d = kv.dims(w.B, w.Hq, w.Hkv, w.S, w.D)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    mass = torch.empty((w.B, w.Hkv, w.S), dtype=torch.float32, device=dev)
    tws = torch.empty(kv.workspace_bytes(kv.OP_FUTURE_TARGET, d, w.window), dtype=torch.uint8,
                      device=dev)
    fws = torch.empty(max(kv.workspace_bytes(kv.OP_FWD_LSE, d), 16), dtype=torch.uint8, device=dev)
    sp = torch.empty((w.B, w.Hkv, w.budget), dtype=torch.int32, device=dev)
    ss = torch.empty((w.B, w.Hkv, w.budget), dtype=torch.float32, device=dev)
    kc = torch.empty((w.B, w.Hkv, w.budget, w.D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)

    def layer(i, ev=None):
        q, k, v = ins[i]
        if ev:
            ev[0].record()
        kv.fwd_lse(q, k, out=lse, workspace=fws)
        if ev:
            ev[1].record()
        kv.future_attn_target(q, k, lse, w.window, agg="sum", out=mass, workspace=tws)
        if ev:
            ev[2].record()
        kv.evict_select(mass, w.n_sink, w.window, w.budget, k, v, out_pos=sp, out_score=ss,
                        out_k=kc, out_v=vc)
        if ev:
            ev[3].record()

    for i in range(warm):
        layer(i % layers)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps * layers)]
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for r in range(reps):
        for i in range(layers):
            layer(i, evs[r * layers + i])
    b.record()
    torch.cuda.synchronize()
    n = reps * layers
    ms_pass = a.elapsed_time(b) / reps
    t_fwd = sum(e[0].elapsed_time(e[1]) for e in evs) / n
    t_tr = sum(e[1].elapsed_time(e[2]) for e in evs) / n
    t_sel = sum(e[2].elapsed_time(e[3]) for e in evs) / n
    f_fwd, f_tr = target_flops(w)
    rows = w.B * w.Hkv
    sg_bytes = rows * (4 * w.S + 8 * w.budget) + rows * 2 * (2 * w.budget * w.D * 2)
    tf = lambda f, ms: f / (ms / 1e3) / 1e12
    keys = layers * w.B * w.Hkv * w.S
    out = {"workload": w.name, "batch": w.B, "seq_len": w.S, "layers": layers, "window": w.window,
           "budget": w.budget, "reps": reps, "ms_per_pass": ms_pass,
           "keys_per_s": keys / (ms_pass / 1e3),
           "per_layer_ms": {"fwd_lse": t_fwd, "future_attn_target": t_tr, "select_gather": t_sel},
           "fwd_lse": {"flops": f_fwd, "tflops": tf(f_fwd, t_fwd),
                       "frac": tf(f_fwd, t_fwd) / MFMA_BF16_PEAK_TFLOPS},
           "future_attn_target": {"flops": f_tr, "tflops": tf(f_tr, t_tr),
                                  "frac": tf(f_tr, t_tr) / MFMA_BF16_PEAK_TFLOPS},
           "select_gather": {"bytes": sg_bytes, "achieved": sg_bytes / (t_sel / 1e3) / 1e9,
                             "unit": "GB/s",
                             "frac": sg_bytes / (t_sel / 1e3) / 1e9 / HBM_PEAK_GBS}}
    del ins
    torch.cuda.empty_cache()
    return out


def decode_bytes_per_step(w, layers):
    """Algorithmic HBM bytes of one decode step over all layers: the whole
    bounded K/V cache read once, the appended K/V rows written, the exiting
    row copied (read + write, upper bound), q read and o written (bf16)."""
    units = w.B * w.Hkv * layers
    cache = units * 2 * w.budget * w.D * 2
    append = units * 2 * w.D * 2
    exit_copy = units * 2 * 2 * w.D * 2
    qo = w.B * layers * w.Hq * w.D * 2 * 2
    return cache + append + exit_copy + qo


def _one_counter(a, ms):
    """Counter bytes of one kernel launched once per `ms`."""
    ba = counter_bytes(a)
    if ba is None:
        return None
    gbs = ba / (ms / 1e3) / 1e9
    return {"bytes": ba, "achieved": gbs, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}


def _pair_counters(a, b, ms):
    """Counter bytes of two kernels launched together once per `ms`."""
    ba, bb = counter_bytes(a), counter_bytes(b)
    if ba is None or bb is None:
        return None
    gbs = (ba + bb) / (ms / 1e3) / 1e9
    return {"bytes": ba + bb, "achieved": gbs, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}


def time_prefix_retention(kv, w, kp, vp, mlp, reps=3):
    """One-shot retention of one layer's prefix (64 x 8 rows of 32768 tokens
    down to the budget): the MLP scorer over every prefix key (one FMA per
    weight and key, fp32 on the vector ALU), selection (reads every score,
    writes positions and scores) and selection + compaction (the gather also
    reads and writes every kept K and V row)."""
    rows = w.B * w.Hkv
    hidden = mlp[0].shape[1]
    score_flops = 2 * rows * w.S * hidden * w.D
    sel_bytes = rows * (4 * w.S + 8 * w.budget)
    gat_bytes = rows * 2 * (2 * w.budget * w.D * 2)
    sc = kv.score_mlp(kp, *mlp)
    outs = kv.evict_select(sc, w.n_sink, w.window, w.budget, kp, vp)

    def t_ms(fn):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_score = t_ms(lambda: kv.score_mlp(kp, *mlp, out=sc))
    t_sel = t_ms(lambda: kv.evict_select(sc, w.n_sink, w.window, w.budget, out_pos=outs[0],
                                         out_score=outs[1]))
    t_both = t_ms(lambda: kv.evict_select(sc, w.n_sink, w.window, w.budget, kp, vp, out_pos=outs[0],
                                          out_score=outs[1], out_k=outs[2], out_v=outs[3]))
    del outs
    gbs = lambda by, ms: by / (ms / 1e3) / 1e9
    tfl = score_flops / (t_score / 1e3) / 1e12
    return {"rows": rows, "seq_len": w.S, "budget": w.budget,
            "score": {"ms": t_score, "flops": score_flops, "achieved": tfl, "unit": "TFLOP/s",
                      "bound": "alu", "peak": FP32_VECTOR_PEAK_TFS,
                      "frac": tfl / FP32_VECTOR_PEAK_TFS},
            "score_select_gather_ms": t_score + t_both,
            "select": {"ms": t_sel, "bytes": sel_bytes, "achieved": gbs(sel_bytes, t_sel),
                       "unit": "GB/s", "frac": gbs(sel_bytes, t_sel) / HBM_PEAK_GBS,
                       "counters": counter_hbm("select_decode_prefix", 1e3 / t_sel)},
            "select_gather": {"ms": t_both, "bytes": sel_bytes + gat_bytes,
                              "achieved": gbs(sel_bytes + gat_bytes, t_both), "unit": "GB/s",
                              "frac": gbs(sel_bytes + gat_bytes, t_both) / HBM_PEAK_GBS,
                              "counters": _pair_counters("select_decode_prefix",
                                                         "gather_decode_prefix", t_both)}}


def bench_decode(kv, steps, layers, seed=5):
    w = synth.DECODE
    dev = torch.device("cuda")
    hidden, delay = w.extra["hidden"], w.extra["delay"]
    B, Hq, Hkv, D, S, bud = w.B, w.Hq, w.Hkv, w.D, w.S, w.budget
    log(f"decode setup: {layers} layers, prefix {S} -> budget {bud}")
    caches = []
    mlps = []
    for layer in range(layers):
        ls = 1000 * 5 + layer
        kp = synth.bf16(synth.normal((B, Hkv, S, D), ls * 3 + 1, dev, w.std))
        vp = synth.bf16(synth.normal((B, Hkv, S, D), ls * 3 + 2, dev, w.std))
        mlp = [t.to(dev) for t in synth.mlp_weights(Hkv, D, hidden, seed=ls)]
        if layer == 0:
            prefix_retention = time_prefix_retention(kv, w, kp, vp, mlp)
        sc = kv.score_mlp(kp, *mlp)
        sp, ss, kc, vc = kv.evict_select(sc, w.n_sink, w.window, bud, kp, vp)
        del kp, vp, sc
        caches.append([kc, vc, sp, ss])
        mlps.append(mlp)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    qs = torch.randn((steps, layers, B, Hq, D), generator=g, device=dev).mul_(w.std).to(torch.bfloat16)
    ks = torch.randn((steps, layers, B, Hkv, D), generator=g, device=dev).mul_(w.std).to(torch.bfloat16)
    vs = torch.randn((steps, layers, B, Hkv, D), generator=g, device=dev).mul_(w.std).to(torch.bfloat16)
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    dd = kv.dims(B, Hq, Hkv, bud, D)
    dws = torch.empty(kv.workspace_bytes(kv.OP_DECODE, dd), dtype=torch.uint8, device=dev)

    def one_step(i, pos):
        for layer in range(layers):
            kc, vc, sp, ss = caches[layer]
            kv.cache_step(kc, vc, sp, ss, ks[i, layer], vs[i, layer], pos, w.n_sink, w.window, delay,
                          mlp=mlps[layer])
            kv.decode_attend(qs[i, layer], kc, vc, sp, out_dtype=torch.bfloat16, want_lse=False,
                             out=o, workspace=dws)

    def one_fused_step(i, pos):
        for layer in range(layers):
            kc, vc, sp, ss = caches[layer]
            kv.decode_step(qs[i, layer], kc, vc, sp, ss, ks[i, layer], vs[i, layer], pos, w.n_sink,
                           w.window, delay, mlp=mlps[layer], out_dtype=torch.bfloat16,
                           want_lse=False, out=o, workspace=dws)

    # attention-only timing of one layer (events on the launch stream)
    ea = torch.cuda.Event(enable_timing=True)
    eb = torch.cuda.Event(enable_timing=True)
    kc, vc, sp, ss = caches[0]
    for _ in range(3):
        kv.decode_attend(qs[0, 0], kc, vc, sp, out_dtype=torch.bfloat16, want_lse=False, out=o,
                         workspace=dws)
    n_att = 50
    ea.record()
    for _ in range(n_att):
        kv.decode_attend(qs[0, 0], kc, vc, sp, out_dtype=torch.bfloat16, want_lse=False, out=o,
                         workspace=dws)
    eb.record()
    torch.cuda.synchronize()
    t_att_ms = ea.elapsed_time(eb) / n_att

    def timed(fn, pos0, label):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i, pos0 + i)
            if (i + 1) % 128 == 0:
                log(f"decode ({label}): {i + 1}/{steps} steps issued")
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1), time.perf_counter() - t0

    # the decode steps continue one sequence: the two-call run takes the
    # positions after the fused run (kvpop_decode_step, the primary figure)
    ms, wall = timed(one_fused_step, S, "fused decode step")
    ms_two, _ = timed(one_step, S + steps, "cache step + attention")

    # the same decode with the delayed stateful mLSTM scorer in place of the
    # MLP: per layer, the scorer takes the new token and scores the exiting
    # one (kvpop_mlstm_step), then kvpop_decode_step with no scorer of its own
    # keeps or drops it and attends.  Random-init scorer per layer (weights
    # N(0, 1/fan_in), forget-gate bias +3, input-gate bias 0); its state
    # starts empty at the first timed step (the per-step work does not depend
    # on the state's contents).
    mls, states = [], []
    for layer in range(layers):
        g = torch.Generator(device=dev)
        g.manual_seed(7000 + layer)
        X = 2 * D
        r = lambda *sh: torch.randn(sh, generator=g, device=dev, dtype=torch.float32)
        mls.append({"wk": r(Hkv, 32, X) / X ** 0.5, "wr": r(Hkv, 32, X) / X ** 0.5,
                    "wv": r(Hkv, 64, X) / X ** 0.5, "wi": r(Hkv, X) / X ** 0.5,
                    "bi": torch.zeros(Hkv, device=dev), "wf": r(Hkv, X) / X ** 0.5,
                    "bf": torch.full((Hkv,), 3.0, device=dev), "wo": r(Hkv, 64) / 8.0,
                    "bo": torch.zeros(Hkv, device=dev)})
        states.append(kv.mlstm_state(B, Hkv, device=dev))

    def one_mlstm_step(i, pos):
        for layer in range(layers):
            kc, vc, sp, ss = caches[layer]
            kv.decode_step_mlstm(qs[i, layer], kc, vc, sp, ss, ks[i, layer], vs[i, layer],
                                 mls[layer], states[layer], pos, w.n_sink, w.window,
                                 out_dtype=torch.bfloat16, want_lse=False, out=o, workspace=dws)

    def one_mlstm_two_calls(i, pos):
        for layer in range(layers):
            kc, vc, sp, ss = caches[layer]
            kv.mlstm_step(ks[i, layer], vs[i, layer], mls[layer], states[layer], pos, w.n_sink,
                          w.window, kc, vc, ss)
            kv.decode_step(qs[i, layer], kc, vc, sp, ss, ks[i, layer], vs[i, layer], pos, w.n_sink,
                           w.window, 0, out_dtype=torch.bfloat16, want_lse=False, out=o,
                           workspace=dws)

    for i in range(2):  # warm-up of the new kernels
        one_mlstm_step(i, S + 2 * steps + i)
    ms_ml, _ = timed(one_mlstm_step, S + 2 * steps + 2, "mLSTM scorer + decode step, one call")
    ms_ml2, _ = timed(one_mlstm_two_calls, S + 3 * steps + 2, "mLSTM scorer, then decode step")
    ml_extra = layers * B * Hkv * (2 * 4 * (64 * 64 + 64 + 4) + 2 * D * 2)  # state r+w, x_u
    sps = steps / (ms / 1e3)
    by = decode_bytes_per_step(w, layers)
    att_bytes = B * Hkv * 2 * bud * D * 2 + B * Hq * D * 2 * 2
    return {
        "workload": w.name, "sequences": B, "layers": layers, "steps": steps, "budget": bud,
        "prefix": S, "delay": delay, "value": sps, "unit": "steps/s", "ms_per_step": ms / steps,
        "wall_s": wall, "bytes_per_step": by,
        "hbm": {"achieved": by * sps / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": by * sps / 1e9 / HBM_PEAK_GBS,
                "counters": counter_hbm("decode_step", sps * layers)},
        "prefix_retention": prefix_retention,
        "entry_point": "kvpop_decode_step",
        "two_calls": {"entry_points": "kvpop_cache_step + kvpop_decode_attend",
                      "value": steps / (ms_two / 1e3), "unit": "steps/s",
                      "ms_per_step": ms_two / steps,
                      "hbm_frac": by * steps / (ms_two / 1e3) / 1e9 / HBM_PEAK_GBS},
        "mlstm_scorer": {"entry_point": "kvpop_decode_step_mlstm",
                         "value": steps / (ms_ml / 1e3), "unit": "steps/s",
                         "ms_per_step": ms_ml / steps, "bytes_per_step": by + ml_extra,
                         "hbm_frac": (by + ml_extra) * steps / (ms_ml / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "two_calls": {"entry_points": "kvpop_mlstm_step + kvpop_decode_step "
                                                       "(no scorer)",
                                       "value": steps / (ms_ml2 / 1e3), "unit": "steps/s"},
                         "note": "scorer state 16.7 KB per (sequence, layer, KV head) read and "
                                 "written per step; random-init weights"},
        "attend_kernel": {"ms": t_att_ms, "bytes": att_bytes,
                          "achieved": att_bytes / (t_att_ms / 1e3) / 1e9, "unit": "GB/s",
                          "frac": att_bytes / (t_att_ms / 1e3) / 1e9 / HBM_PEAK_GBS},
    }


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_target_sample(w, threads, min_seconds, seed):
    """The oracle's target work on a bounded, labelled sample of one layer
    of workload w, scaled to the whole workload.  Rounds of randomly drawn
    normalizer rows (LSE of row d costs d + 1 dot products) and key columns
    (the future mass of key t costs G * (S - t - w) dot products, fed seeded
    stand-in normalizers: the oracle's cost does not depend on their values)
    run until `min_seconds` have passed; each half is scaled by its share of
    the layer's dot products.  Selection is timed on every row of the layer.
    Returns KV-head keys per second over the whole workload (every layer
    costs the same)."""
    import numpy as np

    import oracle

    q, k, _ = synth.attention_inputs(w, seed=seed)
    qf = np.ascontiguousarray(q.float().numpy())
    kf = np.ascontiguousarray(k.float().numpy())
    del q, k
    G = w.Hq // w.Hkv
    r = np.random.default_rng(seed)
    t_rows = t_keys = 0.0
    dots_rows = dots_keys = 0
    n_rows = n_keys = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_seconds:
        bh = int(r.integers(w.B * w.Hkv))
        b, h = divmod(bh, w.Hkv)
        qs = np.ascontiguousarray(qf[b:b + 1, h * G:(h + 1) * G])
        ks = np.ascontiguousarray(kf[b:b + 1, h:h + 1])
        rows = r.integers(0, G * w.S, 64).astype(np.int64)
        a = time.perf_counter()
        oracle.lse(qs, ks, rows=rows, nthreads=threads)
        t_rows += time.perf_counter() - a
        dots_rows += int((rows % w.S + 1).sum())
        n_rows += rows.size
        cols = r.integers(0, w.S, 64).astype(np.int64)
        lse_stand_in = synth.normalizers(1, G, w.S, seed=seed + n_keys).double().numpy()
        a = time.perf_counter()
        oracle.future_mass(qs, ks, lse_stand_in, w.window, cols=cols, nthreads=threads)
        t_keys += time.perf_counter() - a
        dots_keys += int((G * np.clip(w.S - cols - w.window, 0, None)).sum())
        n_keys += cols.size
    # dot products of one layer: LSE rows sum_d (d + 1) per query head;
    # mass sum_t max(0, S - t - w) per query head
    n = max(w.S - w.window, 0)
    layer_rows = w.B * w.Hq * w.S * (w.S + 1) // 2
    layer_keys = w.B * w.Hq * n * (n + 1) // 2
    sc = synth.scores((w.B, w.Hkv, w.S), seed=seed).numpy()
    a = time.perf_counter()
    oracle.select(sc, w.n_sink, w.window, w.budget)
    t_sel = time.perf_counter() - a
    t_layer = t_rows * layer_rows / dots_rows + t_keys * layer_keys / dots_keys + t_sel
    return {"value": w.B * w.Hkv * w.S / t_layer, "unit": "keys/s", "cores": threads,
            "kind": "oracle", "workload": w.name,
            "sample": f"{n_rows} LSE rows and {n_keys} key columns of one {w.name} layer "
                      f"({t_rows + t_keys:.1f} s), each scaled by its share of the layer's dot "
                      f"products, plus selection of all {w.B * w.Hkv} rows ({t_sel:.2f} s)"
                      + ("; every layer costs the same" if w.layers > 1 else ""),
            "scaled_s_per_layer": t_layer}


def cpu_baseline(min_seconds=10.0):
    """The oracle (plain C, double, all host threads) on bounded samples:
    the 36-layer prefill (the headline workload, scaled from sampled rows
    and keys), the skewed 16k batch (the same way), the Qwen3-4B layer's
    whole target work (LSE of all 32 query heads, the future mass of all
    8 x 4096 keys, then selection), and the decode step on a few (sequence,
    layer) units of the bounded-decode workload, scaled to whole steps."""
    import numpy as np

    import oracle

    threads = len(os.sched_getaffinity(0))
    out = cpu_target_sample(synth.QWEN8B, threads, min_seconds, seed=4000)
    out["cpu_model"] = cpu_model()
    out["skewed_long"] = cpu_target_sample(synth.SKEWED, threads, min_seconds / 2, seed=3000)
    w = synth.QWEN4B
    q, k, _ = synth.attention_inputs(w, seed=7)
    qf = np.ascontiguousarray(q.float().numpy())
    kf = np.ascontiguousarray(k.float().numpy())
    reps = 0
    t0 = time.perf_counter()
    while True:
        lse = oracle.lse(qf, kf, nthreads=threads)
        m = oracle.future_mass(qf, kf, lse, w.window, nthreads=threads)
        oracle.select(m.astype(np.float32), w.n_sink, w.window, w.budget)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds / 2:
            break
    keys = w.B * w.Hkv * w.S
    out["layer_step"] = {"value": keys * reps / dt, "unit": "keys/s", "cores": threads,
                         "kind": "oracle", "workload": w.name,
                         "sample": f"{reps} full {w.name} target computations (LSE of {w.Hq} query "
                                   f"heads, future mass of {keys} keys, selection); {dt:.1f} s"}
    # the same layer on one host thread, from a sampled bound (the full
    # layer takes about half a minute on one thread)
    out["layer_step"]["one_thread"] = cpu_target_sample(w, 1, min_seconds / 4, seed=4100)
    out["decode"] = cpu_decode_baseline(threads)
    return out


def cpu_decode_baseline(threads, units=4, steps=16):
    """Oracle decode steps/s on the bounded-decode workload, from `units`
    (sequence, layer) pairs advanced `steps` steps (one cache step with given
    scores and one decode attention each), scaled by the fraction of the
    64 x 36 units of a whole step."""
    import numpy as np

    import oracle

    w = synth.DECODE
    Hq, Hkv, D, bud, S = w.Hq, w.Hkv, w.D, w.budget, w.S
    g = np.random.default_rng(5)
    n_sink, window, delay = w.n_sink, w.window, w.extra["delay"]
    k_sel = bud - n_sink - window

    def bf16_bits(shape):  # N(0, 0.5^2) truncated to bf16 bit patterns
        x = (g.standard_normal(shape) * w.std).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    t_total = 0.0
    for u in range(units):
        # a full cache as the prefix selection leaves it: sinks, the k
        # selected tokens (ascending), the window ring
        sel = np.sort(g.choice(np.arange(n_sink, S - window), k_sel, replace=False))
        pos = np.concatenate([np.arange(n_sink), sel, np.zeros(window, np.int64)])
        ring = np.arange(S - window, S)
        pos[n_sink + k_sel + ring % window] = ring
        sp = np.broadcast_to(pos.astype(np.int32), (1, Hkv, bud)).copy()
        ss = g.standard_normal((1, Hkv, bud)).astype(np.float32)
        state = {"slot_pos": sp, "slot_score": ss, "kc": bf16_bits((1, Hkv, bud, D)),
                 "vc": bf16_bits((1, Hkv, bud, D))}
        for i in range(steps):
            kn = bf16_bits((1, Hkv, D))
            vn = bf16_bits((1, Hkv, D))
            sr = g.standard_normal((1, Hkv)).astype(np.float32)
            qn = g.standard_normal((1, Hq, D)).astype(np.float32)
            t0 = time.perf_counter()
            oracle.cache_step(state, kn, vn, sr, n_sink, window, delay, S + i)
            oracle.decode_attend(qn, oracle.bf16_bits_to_f32(state["kc"]),
                                 oracle.bf16_bits_to_f32(state["vc"]), state["slot_pos"],
                                 nthreads=threads)
            t_total += time.perf_counter() - t0
    per_unit_step = t_total / (units * steps)
    whole = w.B * 36 * per_unit_step
    return {"value": 1.0 / whole, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"{units} (sequence, layer) units x {steps} steps of the {w.name} workload "
                      f"(cache step with given scores + decode attention), {t_total:.1f} s, scaled "
                      f"by 64 x 36 units per step"}


def sources_digest(names=TRAFFIC_SOURCES):
    """SHA-256 of kernel sources with comments and blank lines removed, so
    that only a change of code invalidates recorded counters."""
    import hashlib
    import re

    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "future_attention_scoring_kvpop_amd", "csrc", name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()


def traffic_bytes():
    """The recorded HBM traffic of the target call, or None when the kernel
    code differs from the code it was measured on."""
    if TRAFFIC is None or sources_digest() != TRAFFIC["sha256"]:
        return None
    return TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]


def counter_bytes(name):
    """HBM bytes per dispatch recorded for one of COUNTERS, or None when the
    kernel's sources differ from those the counters were taken on."""
    c = COUNTERS[name]
    sha = COUNTER_SHA["decode" if name == "decode_step" else "select"]
    if sources_digest(c["sources"]) != sha:
        return None
    return 2.0 * c["fetch_kib"] * 1024 + c["write_kib"] * 1024


def counter_hbm(name, dispatches_per_s):
    """{bytes, achieved GB/s, frac} from the recorded counters at a measured
    dispatch rate (None when the counters are stale)."""
    by = counter_bytes(name)
    if by is None:
        return None
    gbs = by * dispatches_per_s / 1e9
    return {"bytes_per_dispatch": by, "achieved": gbs, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "per": COUNTERS[name]["per"]}


def calibrate_copy(mib):
    """A plain device copy of known size for scaling the FETCH_SIZE and
    WRITE_SIZE counters: 5 launches of torch's copy kernel over `mib` MiB."""
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


LEGS = ("prefill", "layer", "variants", "retention", "sparse", "skewed", "attn_out",
        "sparse_long", "decode", "cpu")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed steps of the 36-layer prefill")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--prefill-layers", type=int, default=36,
                    help="layers of the headline step (fewer only for profiling runs)")
    ap.add_argument("--layer-steps", type=int, default=20)
    ap.add_argument("--layer-warmup", type=int, default=50)
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--decode-layers", type=int, default=36)
    ap.add_argument("--only", default="", help="comma-separated legs to run: " + ",".join(LEGS))
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the skewed 16k batch and the 32k sparse-normalizer layer")
    ap.add_argument("--calibrate-copy", type=int, metavar="MIB", default=0,
                    help="only run a plain copy of MIB MiB (counter calibration)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the KVpop hot path is sharded by (batch, KV head) with no "
              "communication, and the library runs on one MI355X; use --gpus 1.", flush=True)
        sys.exit(2)

    if a.calibrate_copy:
        calibrate_copy(a.calibrate_copy)
        return
    legs = set(a.only.split(",")) if a.only else set(LEGS)
    bad = legs - set(LEGS)
    if bad:
        ap.error(f"unknown legs {sorted(bad)}")
    if a.no_decode:
        legs.discard("decode")
    if a.no_cpu:
        legs.discard("cpu")
    if a.no_long:
        legs -= {"skewed", "sparse_long"}

    import dataclasses

    import future_attention_scoring_kvpop_amd as kv

    if not os.path.exists(kv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    torch.cuda.set_device(0)

    w = synth.QWEN8B
    if a.prefill_layers != w.layers:
        w = dataclasses.replace(w, layers=a.prefill_layers)
    out = {"metric": METRIC, "value": None, "unit": "keys/s", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": w.name, "layers": w.layers, "batch": w.B, "q_heads": w.Hq,
                      "kv_heads": w.Hkv, "head_dim": w.D, "seq_len": w.S, "window": w.window,
                      "sinks": w.n_sink, "budget": w.budget, "aggregation": "sum",
                      "rope_theta": synth.ROPE_THETA,
                      "step": "per layer: fwd_lse + future_attn_target + evict_select(+gather) + "
                              "decode_step (cache step with delayed MLP score + decode attention)"}}
    if "prefill" in legs:
        log(f"{w.name}: {a.warmup} warm-up + {a.steps} timed steps of {w.layers} layers")
        pre = bench_prefill_step(kv, w, a.steps, a.warmup)
        achieved = pre["f_target"] / (pre["t_target_ms"] / 1e3) / 1e12
        out["value"] = pre["keys_per_s"]
        out["ms_per_step"] = pre["ms_per_step"]
        out["roofline"] = {"bound": "mfma",
                           "kernel": "kvpop_future_attn_target (transposed pass + merge)",
                           "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic_bytes(),
                           "flops_per_launch": pre["f_target"], "ms_per_launch": pre["t_target_ms"]}
        out["prefill_36_layers"] = {k_: v_ for k_, v_ in pre.items()
                                    if k_ not in ("t_target_ms", "f_target")}
        if w.layers != 36:
            out["reduced"] = True
        log(f"{w.name}: {pre['ms_per_step']:.2f} ms per step, {out['value']:.4g} keys/s, "
            f"target {achieved / MFMA_BF16_PEAK_TFLOPS:.3f} of peak")
    if legs & {"layer", "variants", "retention", "sparse"}:
        log(f"layer step: {a.layer_warmup} warmup + {a.layer_steps} timed")
        st, ms, t_tr, brk, f_fwd, f_tr = bench_target(kv, a.layer_steps, a.layer_warmup)
        wl = st.w
        tf = lambda f, t: f / (t / 1e3) / 1e12
        out["layer_step"] = {
            "workload": wl.name, "ms_per_step": ms, "keys_per_s": wl.B * wl.Hkv * wl.S / (ms / 1e3),
            "step": "fwd_lse + future_attn_target + evict_select(+gather) + cache_step + "
                    "decode_attend",
            "fwd_lse": {"ms": brk["fwd_lse"], "tflops": tf(f_fwd, brk["fwd_lse"]),
                        "frac": tf(f_fwd, brk["fwd_lse"]) / MFMA_BF16_PEAK_TFLOPS},
            "future_attn_target": {"ms": t_tr, "tflops": tf(f_tr, t_tr),
                                   "frac": tf(f_tr, t_tr) / MFMA_BF16_PEAK_TFLOPS},
            "select_gather_decode": {"ms": brk["select_gather_decode"]},
            "instrumented_ms_per_step": brk["ms_per_step"],
            "note": "fwd_lse and select_gather_decode from a second loop with events around every "
                    "pass; future_attn_target from the timed steps"}
        if "variants" in legs:
            out["layer_step"]["target_variants"] = bench_target_variants(kv, st)
        if "retention" in legs:
            out["layer_step"]["retention"] = bench_retention(kv, st)
        if "sparse" in legs:
            log("sparse normalizer: running top-k mask, sparse causal pass, transposed pass")
            out["sparse_normalizer"] = bench_sparse(kv, st)
        del st
        torch.cuda.empty_cache()
    if "attn_out" in legs:
        log("attention output of the main pass: 4k layer and one 32k layer")
        out["attention_output"] = {"qwen3-4b-layer": bench_attention_output(kv, synth.QWEN4B, reps=20),
                                   "qwen3-8b-prefill-layer": bench_attention_output(kv, synth.QWEN8B)}
    if "skewed" in legs:
        log("skewed-long: 4 x 16384, 3 warm-up and 4 timed passes")
        out["skewed_long"] = bench_prefill(kv, synth.SKEWED, reps=4, warm=3)
    if "sparse_long" in legs:
        log("sparse normalizer on one 32k-prefill layer")
        out["sparse_normalizer_32k_layer"] = bench_sparse_long(kv, synth.QWEN8B)
    if "decode" in legs:
        log(f"decode: {a.decode_steps} steps x {a.decode_layers} layers")
        out["decode"] = bench_decode(kv, a.decode_steps, a.decode_layers)
        if a.decode_layers != 36 or a.decode_steps != 512:
            out["decode"]["reduced"] = True
    if "cpu" in legs:
        log("cpu baseline: oracle on bounded samples")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
