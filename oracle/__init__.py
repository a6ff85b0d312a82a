"""CPU oracle for the KVpop hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``future_attention_scoring_kvpop_amd``) and never imports it.

Everything here is a thin numpy/ctypes wrapper around ``kvpop_oracle.c``
(plain C, double accumulation), plus ``gather`` which is a plain numpy
indexing copy.  ``oracle.brute`` holds the dense S x S brute force that pins
this oracle at tiny sizes.

Method source: "KVpop -- Key-Value Cache Compression with Predictive Online
Pruning" (arXiv 2607.05061v2), paperlayer.ai summary: App. D.1-D.4 (target;
D.3 sparse normalizer; D.4 and App. I the main pass's attention output), App. C.1-C.2 (running top-k mask and its cutoffs), App. A and E.3-E.4 (the
delayed stateful mLSTM scorer),
App. B.1-B.2 (aggregation, count normalisation), Sec. 3 and App. C.1
(fixed-budget retention), App. E.2 and E.4 (scorer, delayed readout).

Parity status per function (see the tests under tests/test_oracle_*.py):
  lse, future_mass, select, gather, decode_attend, mlp_score, cache_step,
  running_topk, lse_sparse, mlstm_scores, attn_out: pinned (brute force, closed forms, invariants,
  hand-worked fixtures).
"""
import ctypes
import math
import os

import numpy as np

from . import build as _build

_LIB = None

AGG = {"sum": 0, "mean": 1, "max": 2}


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_long
        Dd = ctypes.c_double
        lib.oracle_lse.argtypes = [I, I, I, I, I, Dd, P, P, L, P, P, I]
        lib.oracle_future_mass.argtypes = [I, I, I, I, I, Dd, P, P, P, I, I, I, I, L, P, P, P, I]
        lib.oracle_select.argtypes = [I, I, I, I, I, I, P, P, P]
        lib.oracle_decode_attend.argtypes = [I, I, I, I, I, Dd, P, P, P, P, P, P, I]
        lib.oracle_mlp_score.argtypes = [I, I, I, I, I, P, P, P, P, P, P]
        lib.oracle_cache_step.argtypes = [I, I, I, I, I, I, I, I, P, P, P, P, P, P, P]
        lib.oracle_running_topk.argtypes = [I, I, I, I, I, I, P, P, P, P]
        lib.oracle_lse_sparse.argtypes = [I, I, I, I, I, Dd, P, P, P, P, I, I, I, L, P, P, I]
        lib.oracle_mlstm_scores.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.oracle_attn_out.argtypes = [I, I, I, I, I, Dd, P, P, P, P, P, I, I, I, L, P, P, P, P, I]
        for f in ("oracle_lse", "oracle_future_mass", "oracle_select", "oracle_decode_attend",
                  "oracle_mlp_score", "oracle_cache_step", "oracle_running_topk",
                  "oracle_lse_sparse", "oracle_mlstm_scores", "oracle_attn_out"):
            getattr(lib, f).restype = ctypes.c_int
        _LIB = lib
    return _LIB


def _threads(n):
    if n is not None:
        return int(n)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def bf16_bits_to_f32(bits):
    """Exact widening of raw bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def default_scale(D):
    return 1.0 / math.sqrt(D)


def lse(q, k, scale=None, rows=None, nthreads=None):
    """Dense causal natural-log normalizer LSE[b, g, d] (App. D.1, D.4).

    q [B,Hq,S,D], k [B,Hkv,S,D] (float values, e.g. bf16 widened exactly).
    rows: optional flat indices (b*Hq + g)*S + d; returns the full [B,Hq,S]
    array when rows is None, else a vector over rows.
    """
    q = _f32(q)
    k = _f32(k)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    sc = default_scale(D) if scale is None else float(scale)
    if rows is None:
        n = B * Hq * S
        rp = None
        out = np.empty(n, np.float64)
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
        rp = _ptr(rows)
        out = np.empty(n, np.float64)
    _check(_lib().oracle_lse(B, Hq, Hkv, S, D, sc, _ptr(q), _ptr(k), n, rp, _ptr(out),
                             _threads(nthreads)), "lse")
    return out.reshape(B, Hq, S) if rows is None else out


def future_mass(q, k, lse_arr, window, lookahead=-1, agg="sum", count_normalize=False,
                cols=None, per_head=False, scale=None, nthreads=None):
    """Future-attention mass per key (App. D.1-D.2, B.1-B.2).

    lse_arr: [B,Hq,S] float64 normalizers (the oracle's own).  Returns mass
    [B,Hkv,S] (or a vector over ``cols``, flat (b*Hkv + h)*S + t) and, with
    per_head=True, also the per-query-head mass [..., G].
    """
    q = _f32(q)
    k = _f32(k)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = default_scale(D) if scale is None else float(scale)
    l64 = np.ascontiguousarray(lse_arr, dtype=np.float64)
    assert l64.shape == (B, Hq, S)
    if cols is None:
        n = B * Hkv * S
        cp = None
    else:
        cols = np.ascontiguousarray(cols, dtype=np.int64)
        n = cols.size
        cp = _ptr(cols)
    mass = np.empty(n, np.float64)
    ph = np.empty((n, G), np.float64) if per_head else None
    _check(_lib().oracle_future_mass(B, Hq, Hkv, S, D, sc, _ptr(q), _ptr(k), _ptr(l64),
                                     int(window), int(lookahead), AGG[agg], int(bool(count_normalize)),
                                     n, cp, _ptr(mass), _ptr(ph) if per_head else None,
                                     _threads(nthreads)), "future_mass")
    if cols is None:
        mass = mass.reshape(B, Hkv, S)
        if per_head:
            ph = ph.reshape(B, Hkv, S, G)
    return (mass, ph) if per_head else mass


def select(scores, n_sink, window, budget):
    """Fixed-budget retention and canonical slot layout (Sec. 3, App. C.1, App. F).

    scores [B,Hkv,S] float32.  Returns (slot_pos int32 [B,Hkv,budget],
    slot_score float32 [B,Hkv,budget]; -inf in empty slots).
    """
    sc = _f32(scores)
    B, Hkv, S = sc.shape
    sp = np.empty((B, Hkv, budget), np.int32)
    ss = np.empty((B, Hkv, budget), np.float32)
    _check(_lib().oracle_select(B, Hkv, S, int(n_sink), int(window), int(budget), _ptr(sc),
                                _ptr(sp), _ptr(ss)), "select")
    return sp, ss


def running_topk(scores, n_sink, window, budget, log_decay=None):
    """Running top-k retention mask (App. C.1) with Fenwick-tree cutoffs
    (App. C.2) and per-head decay as static priorities (Sec. 3 teacher
    policy, App. B.3).

    scores [B,Hkv,S] float32; log_decay: None or [Hkv] float32 (-ln gamma_h).
    Returns (keep_until int32 [B,Hkv,S], cutoff int32 [B,Hkv,S]): key t is
    retained for queries t <= d < keep_until[t]; cutoff[d] is the k-th best
    token of the pool at query d, or -1.
    """
    sc = _f32(scores)
    B, Hkv, S = sc.shape
    ld = None if log_decay is None else _f32(log_decay).reshape(Hkv)
    until = np.empty((B, Hkv, S), np.int32)
    cut = np.empty((B, Hkv, S), np.int32)
    _check(_lib().oracle_running_topk(B, Hkv, S, int(n_sink), int(window), int(budget), _ptr(sc),
                                      None if ld is None else _ptr(ld), _ptr(until), _ptr(cut)),
           "running_topk")
    return until, cut


def lse_sparse(q, k, scores, n_sink, window, budget, log_decay=None, scale=None, rows=None,
               nthreads=None):
    """Sparse log-normalizer (App. D.3) over the retained set R_d of the
    running top-k mask (App. C.1), built per query row from its definition.
    Same shapes and ``rows`` convention as ``lse``."""
    q = _f32(q)
    k = _f32(k)
    sc = _f32(scores)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    assert sc.shape == (B, Hkv, S)
    ld = None if log_decay is None else _f32(log_decay).reshape(Hkv)
    s_ = default_scale(D) if scale is None else float(scale)
    if rows is None:
        n = B * Hq * S
        rp = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
        rp = _ptr(rows)
    out = np.empty(n, np.float64)
    _check(_lib().oracle_lse_sparse(B, Hq, Hkv, S, D, s_, _ptr(q), _ptr(k), _ptr(sc),
                                    None if ld is None else _ptr(ld), int(n_sink), int(window),
                                    int(budget), n, rp, _ptr(out), _threads(nthreads)),
           "lse_sparse")
    return out.reshape(B, Hq, S) if rows is None else out


def attn_out(q, k, v, scores=None, n_sink=0, window=0, budget=0, log_decay=None, scale=None,
             rows=None, want_abs=True, nthreads=None):
    """Attention output of the main pass (App. D.4 first step; App. I, the
    sparse student attention over the fixed-budget mask of App. C.1).

    q [B,Hq,S,D], k, v [B,Hkv,S,D] (float values).  scores None: dense
    causal rows R_d = [0, d]; else fp32 [B,Hkv,S] with n_sink, window,
    budget (and log_decay) give the running top-k mask's R_d.  Returns
    (o, o_abs, lse): o[..., c] = sum_{t in R_d} p_dt v_t[c], o_abs the same
    with |v_t[c]| (None unless want_abs), lse the row's natural-log
    normalizer; shapes [B,Hq,S,D] / [B,Hq,S], or [n,D] / [n] over ``rows``.
    """
    q = _f32(q)
    k = _f32(k)
    v = _f32(v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, S, D) and v.shape == k.shape
    sc = None if scores is None else _f32(scores)
    if sc is not None:
        assert sc.shape == (B, Hkv, S)
    ld = None if log_decay is None else _f32(log_decay).reshape(Hkv)
    s_ = default_scale(D) if scale is None else float(scale)
    if rows is None:
        n = B * Hq * S
        rp = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.size
        rp = _ptr(rows)
    o = np.empty((n, D), np.float64)
    oa = np.empty((n, D), np.float64) if want_abs else None
    ls = np.empty(n, np.float64)
    _check(_lib().oracle_attn_out(B, Hq, Hkv, S, D, s_, _ptr(q), _ptr(k), _ptr(v),
                                  None if sc is None else _ptr(sc),
                                  None if ld is None else _ptr(ld), int(n_sink), int(window),
                                  int(budget), n, rp, _ptr(ls), _ptr(o),
                                  None if oa is None else _ptr(oa), _threads(nthreads)),
           "attn_out")
    if rows is None:
        o = o.reshape(B, Hq, S, D)
        oa = None if oa is None else oa.reshape(B, Hq, S, D)
        ls = ls.reshape(B, Hq, S)
    return o, oa, ls


MLSTM_KEYS = ("wk", "wr", "wv", "wi", "bi", "wf", "bf", "wo", "bo")


def mlstm_scores(keys, values, params, window, want_state=False):
    """Delayed stateful mLSTM scores (App. A, E.1, E.3, E.4).

    keys, values [B,Hkv,n,D] (float values); params: dict of the headwise
    weights (MLSTM_KEYS; Wk, Wr [Hkv,P,2D], Wv [Hkv,E,2D], wi, wf [Hkv,2D],
    bi, bf, bo [Hkv], wo [Hkv,E]).  Token u is read out once token u + w has
    entered the state; returns scores [B,Hkv,n] float64 (NaN where never read
    out) and, with want_state, the final (C [B,Hkv,E,2P], n [B,Hkv,2P],
    m [B,Hkv]).
    """
    k = _f32(keys)
    v = _f32(values)
    B, Hkv, n, D = k.shape
    pr = {name: _f32(params[name]) for name in MLSTM_KEYS}
    P = pr["wk"].shape[1]
    E = pr["wv"].shape[1]
    F = 2 * P
    sc = np.empty((B, Hkv, n), np.float64)
    st = np.empty((B, Hkv, E * F + F + 1), np.float64) if want_state else None
    _check(_lib().oracle_mlstm_scores(B, Hkv, n, D, P, E, int(window), _ptr(k), _ptr(v),
                                      *[_ptr(pr[name]) for name in MLSTM_KEYS], _ptr(sc),
                                      None if st is None else _ptr(st)), "mlstm_scores")
    if not want_state:
        return sc
    return sc, (st[..., :E * F].reshape(B, Hkv, E, F), st[..., E * F:E * F + F], st[..., -1])


def gather(x, slot_pos):
    """Compaction (Sec. 3: attention only over the retained set).

    x [B,Hkv,S,D] (any dtype, e.g. raw bf16 bits), slot_pos [B,Hkv,budget].
    Returns x[b,h,slot_pos] with all-zero rows where slot_pos < 0.
    """
    B, Hkv, S, D = x.shape
    sp = np.asarray(slot_pos)
    out = np.zeros(sp.shape + (D,), dtype=x.dtype)
    for b in range(B):
        for h in range(Hkv):
            valid = sp[b, h] >= 0
            out[b, h, valid] = x[b, h, sp[b, h, valid]]
    return out


def decode_attend(q, kc, vc, slot_pos, scale=None, nthreads=None):
    """Decode attention over retained slots (Sec. 3, App. C.1).

    q [B,Hq,D], kc/vc [B,Hkv,n_slots,D] float values, slot_pos [B,Hkv,n_slots].
    Returns (o float64 [B,Hq,D], lse float64 [B,Hq]).
    """
    q = _f32(q)
    kc = _f32(kc)
    vc = _f32(vc)
    sp = np.ascontiguousarray(slot_pos, dtype=np.int32)
    B, Hq, D = q.shape
    Hkv, n_slots = kc.shape[1], kc.shape[2]
    sc = default_scale(D) if scale is None else float(scale)
    o = np.empty((B, Hq, D), np.float64)
    ls = np.empty((B, Hq), np.float64)
    _check(_lib().oracle_decode_attend(B, Hq, Hkv, n_slots, D, sc, _ptr(q), _ptr(kc), _ptr(vc),
                                       _ptr(sp), _ptr(o), _ptr(ls), _threads(nthreads)), "decode")
    return o, ls


def mlp_score(keys, w1, b1, w2, b2):
    """Headwise MLP scorer on keys (App. E.2): float64 [B,Hkv,n_tok]."""
    keys = _f32(keys)
    B, Hkv, n, D = keys.shape
    hidden = w1.shape[1]
    w1 = _f32(w1)
    b1 = _f32(b1)
    w2 = _f32(w2)
    b2 = _f32(b2)
    assert w1.shape == (Hkv, hidden, D) and b1.shape == (Hkv, hidden)
    assert w2.shape == (Hkv, hidden) and b2.shape == (Hkv,)
    out = np.empty((B, Hkv, n), np.float64)
    _check(_lib().oracle_mlp_score(B, Hkv, n, D, hidden, _ptr(keys), _ptr(w1), _ptr(b1),
                                   _ptr(w2), _ptr(b2), _ptr(out)), "mlp_score")
    return out


def cache_step(state, k_new_bits, v_new_bits, scores_r, n_sink, window, delay, pos_q):
    """One bounded-cache decode step, in place (Sec. 3; App. C.1, E.4).

    state: dict with 'kc', 'vc' (uint16 [B,Hkv,budget,D] raw bf16 bits),
    'slot_pos' (int32 [B,Hkv,budget]) and 'slot_score' (float32).
    scores_r: float32 [B,Hkv], the score of token pos_q - delay.
    """
    kc, vc, sp, ss = state["kc"], state["vc"], state["slot_pos"], state["slot_score"]
    for a, dt in ((kc, np.uint16), (vc, np.uint16), (sp, np.int32), (ss, np.float32)):
        assert a.dtype == dt and a.flags.c_contiguous
    B, Hkv, budget, D = kc.shape
    kn = np.ascontiguousarray(k_new_bits, dtype=np.uint16)
    vn = np.ascontiguousarray(v_new_bits, dtype=np.uint16)
    sr = _f32(scores_r)
    _check(_lib().oracle_cache_step(B, Hkv, D, int(n_sink), int(window), budget, int(delay),
                                    int(pos_q), _ptr(kn), _ptr(vn), _ptr(sr), _ptr(kc), _ptr(vc),
                                    _ptr(sp), _ptr(ss)), "cache_step")
    return state
