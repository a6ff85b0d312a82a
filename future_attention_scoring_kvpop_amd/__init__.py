"""libkvpop Python binding: argument marshalling over the C ABI in include/kvpop.h.

Every step of the hot path runs in the HIP kernels of ``libkvpop.so``; this
module only turns torch tensors into device pointers, allocates outputs with
torch (device memory is torch's plumbing) and passes torch's current stream.
There is no fallback: if the library is not built, every call raises.

KVpop (arXiv 2607.05061v2), paperlayer.ai summary: App. D.1-D.4 (future
attention target), App. B.1-B.2 (aggregation, count normalisation), Sec. 3
and App. C.1 (fixed-budget retention), App. E.2 and E.4 (scorer, delayed
readout).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvpop.so")

OK = 0
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
          3: "workspace too small", 4: "device error"}
AGG = {"sum": 0, "mean": 1, "max": 2}
OP_FUTURE_TARGET = 0
OP_DECODE = 1
OP_FWD_LSE = 2
OP_FWD_LSE_SPARSE = 3
OP_FWD_ATTN = 4

EXPORTS = ("kvpop_abi_version", "kvpop_status_string", "kvpop_workspace_bytes", "kvpop_fwd_lse",
           "kvpop_future_attn_target", "kvpop_evict_select", "kvpop_decode_attend",
           "kvpop_score_mlp", "kvpop_cache_step", "kvpop_decode_step", "kvpop_running_topk",
           "kvpop_fwd_lse_sparse", "kvpop_mlstm_step", "kvpop_decode_step_mlstm",
           "kvpop_decode_attend_noalloc", "kvpop_running_topk_workspace_bytes")
DECODE_NOALLOC_SCRATCH_BYTES = 8 << 20


class KvpopError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: {STATUS.get(status, status)} (status {status})")
        self.status = status


class MlstmWeights(ctypes.Structure):
    _fields_ = [("feat", ctypes.c_int), ("vdim", ctypes.c_int)] + [
        (n, ctypes.c_void_p) for n in ("wk", "wr", "wv", "wi", "bi", "wf", "bf", "wo", "bo")]


MLSTM_STATE_FLOATS = 64 * 64 + 64 + 4


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int), ("n_q_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int),
                ("seq_len", ctypes.c_int), ("head_dim", ctypes.c_int), ("scale", ctypes.c_float)]


_lib = None


def lib():
    """The loaded libkvpop.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkvpop.so not built at {LIB_PATH}: run __graft_entry__.build() "
                               "or python future_attention_scoring_kvpop_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        DP = ctypes.POINTER(Dims)
        sig = {
            "kvpop_abi_version": (I, []),
            "kvpop_status_string": (ctypes.c_char_p, [I]),
            "kvpop_workspace_bytes": (Z, [I, DP, I]),
            "kvpop_fwd_lse": (I, [DP, P, P, P, P, P, I, P, Z, P]),
            "kvpop_running_topk": (I, [I, I, I, I, I, I, P, P, P, P, P, Z, P]),
            "kvpop_running_topk_workspace_bytes": (Z, [I, I, I, I]),
            "kvpop_mlstm_step": (I, [I, I, I, I, I, I, I, P, P, P, P, ctypes.POINTER(MlstmWeights),
                                     P, P, P]),
            "kvpop_decode_step_mlstm": (I, [DP, I, I, I, P, P, ctypes.POINTER(MlstmWeights), P, P, P,
                                            P, P, P, P, I, P, P, Z, P]),
            "kvpop_fwd_lse_sparse": (I, [DP, P, P, P, P, I, P, P, I, P, Z, P]),
            "kvpop_future_attn_target": (I, [DP, P, P, P, I, I, I, I, P, P, P, Z, P]),
            "kvpop_evict_select": (I, [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P]),
            "kvpop_decode_attend": (I, [DP, P, P, P, P, P, I, P, P, Z, P]),
            "kvpop_decode_attend_noalloc": (I, [DP, P, P, P, P, P, I, P, P]),
            "kvpop_score_mlp": (I, [I, I, I, I, I, P, P, P, P, P, P, P]),
            "kvpop_cache_step": (I, [I, I, I, I, I, I, I, I, P, P, P, P, P, P, I, P, P, P, P, P, P]),
            "kvpop_decode_step": (I, [DP, I, I, I, I, P, P, P, P, P, P, I, P, P, P, P, P, P, P, I, P,
                                      P, Z, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, st):
    if st != OK:
        raise KvpopError(fn, st)


def _need(t, dtype, name, ndim=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {t.dim()}")


def dims(B, Hq, Hkv, S, D, scale=0.0):
    return Dims(B, Hq, Hkv, S, D, float(scale))


def workspace_bytes(op, d, window=0):
    return int(lib().kvpop_workspace_bytes(op, ctypes.byref(d), int(window)))


def _attn_out(q, v, k, out_o, out_dtype):
    """The output buffer of the main pass, or None without v."""
    if v is None:
        if out_o is not None:
            raise ValueError("out_o needs v")
        return None
    _need(v, torch.bfloat16, "v", 4)
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError("v shape mismatch")
    o = out_o if out_o is not None else torch.empty(q.shape, dtype=out_dtype, device=q.device)
    if o.dtype not in (torch.float32, torch.bfloat16) or tuple(o.shape) != tuple(q.shape):
        raise ValueError("o: expected fp32 or bf16 of q's shape")
    _need(o, o.dtype, "o")
    return o


def fwd_lse(q, k, scale=0.0, out=None, workspace=None, v=None, out_o=None,
            out_dtype=torch.float32):
    """Dense causal log-normalizers LSE [B,Hq,S] fp32 (App. D.1, D.4); with
    v [B,Hkv,S,D] also the causal attention output O [B,Hq,S,D] (fp32 or
    bf16 per out_dtype), returned as (lse, o)."""
    _need(q, torch.bfloat16, "q", 4)
    _need(k, torch.bfloat16, "k", 4)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, S, D):
        raise ValueError("k shape mismatch")
    lse = out if out is not None else torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _need(lse, torch.float32, "lse")
    o = _attn_out(q, v, k, out_o, out_dtype)
    d = dims(B, Hq, Hkv, S, D, scale)
    nbytes = workspace_bytes(OP_FWD_ATTN if v is not None else OP_FWD_LSE, d)
    ws = workspace if workspace is not None else (
        torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None)
    st = lib().kvpop_fwd_lse(ctypes.byref(d), _p(q), _p(k), _p(v), _p(lse), _p(o),
                             1 if o is not None and o.dtype == torch.bfloat16 else 0, _p(ws),
                             0 if ws is None else ws.numel() * ws.element_size(), _stream())
    _check("kvpop_fwd_lse", st)
    return lse if o is None else (lse, o)


def running_topk(scores, n_sink, window, budget, log_decay=None, want_cutoff=True, out=None,
                 out_cutoff=None, workspace=None):
    """Running top-k retention mask (App. C.1) and its per-query cutoffs
    (App. C.2) with per-head decay priorities (Sec. 3, App. B.3).

    scores fp32 [B,Hkv,S]; log_decay None or fp32 [Hkv].  Returns
    (keep_until int32 [B,Hkv,S], cutoff int32 [B,Hkv,S] or None).
    """
    _need(scores, torch.float32, "scores", 3)
    B, Hkv, S = scores.shape
    if log_decay is not None:
        _need(log_decay, torch.float32, "log_decay")
        if log_decay.numel() != Hkv:
            raise ValueError("log_decay: expected one value per KV head")
    until = out if out is not None else torch.empty((B, Hkv, S), dtype=torch.int32,
                                                    device=scores.device)
    _need(until, torch.int32, "keep_until")
    cut = None
    if want_cutoff:
        cut = out_cutoff if out_cutoff is not None else torch.empty_like(until)
        _need(cut, torch.int32, "cutoff")
    need = lib().kvpop_running_topk_workspace_bytes(B, Hkv, S, int(n_sink))
    ws = workspace
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        ws = torch.empty(need, dtype=torch.uint8, device=scores.device)
    st = lib().kvpop_running_topk(B, Hkv, S, int(n_sink), int(window), int(budget), _p(scores),
                                  _p(log_decay), _p(until), _p(cut), _p(ws) if need else None,
                                  need, _stream())
    _check("kvpop_running_topk", st)
    return until, cut


def mlstm_state(B, Hkv, device="cuda"):
    """An empty mLSTM scorer state [B,Hkv,MLSTM_STATE_FLOATS]: C = 0, n = 0, m = -inf."""
    st = torch.zeros((B, Hkv, MLSTM_STATE_FLOATS), dtype=torch.float32, device=device)
    st[..., 64 * 64 + 64] = float("-inf")
    return st


def mlstm_step(k_new, v_new, params, state, pos_q, n_sink, window, k_cache=None, v_cache=None,
               slot_score=None):
    """One step of the delayed stateful mLSTM scorer (App. A, E.1, E.3, E.4):
    token pos_q enters the state; with slot_score (and the caches), token
    pos_q - w is read out into its ring slot's score.  params: dict of fp32
    device tensors wk, wr [Hkv,32,2D], wv [Hkv,64,2D], wi, wf [Hkv,2D],
    bi, bf, bo [Hkv], wo [Hkv,64]."""
    _need(k_new, torch.bfloat16, "k_new", 3)
    _need(v_new, torch.bfloat16, "v_new", 3)
    _need(state, torch.float32, "state", 3)
    B, Hkv, D = k_new.shape
    budget = 0
    if slot_score is not None:
        _need(slot_score, torch.float32, "slot_score", 3)
        _need(k_cache, torch.bfloat16, "k_cache", 4)
        _need(v_cache, torch.bfloat16, "v_cache", 4)
        budget = slot_score.shape[-1]
    elif k_cache is not None:
        budget = k_cache.shape[2]
    for n in ("wk", "wr", "wv", "wi", "bi", "wf", "bf", "wo", "bo"):
        _need(params[n], torch.float32, n)
    w = MlstmWeights(params["wk"].shape[1], params["wv"].shape[1],
                     *[params[n].data_ptr() for n in ("wk", "wr", "wv", "wi", "bi", "wf", "bf", "wo", "bo")])
    st = lib().kvpop_mlstm_step(B, Hkv, D, int(n_sink), int(window),
                                int(budget) if budget else int(n_sink) + int(window), int(pos_q),
                                _p(k_new), _p(v_new), _p(k_cache), _p(v_cache), ctypes.byref(w),
                                _p(state), _p(slot_score), _stream())
    _check("kvpop_mlstm_step", st)


def _mlstm_weights(params):
    names = ("wk", "wr", "wv", "wi", "bi", "wf", "bf", "wo", "bo")
    for n in names:
        _need(params[n], torch.float32, n)
    return MlstmWeights(params["wk"].shape[1], params["wv"].shape[1],
                        *[params[n].data_ptr() for n in names])


def decode_step_mlstm(q, k_cache, v_cache, slot_pos, slot_score, k_new, v_new, params, state,
                      pos_q, n_sink, window, out_dtype=torch.float32, want_lse=True, scale=0.0,
                      out=None, out_lse=None, workspace=None):
    """mlstm_step, cache_step with no scorer and decode_attend in one call
    (App. E.3-E.4, Sec. 3, App. C.1): o [B,Hq,D], lse [B,Hq]."""
    _need(q, torch.bfloat16, "q", 3)
    _need(k_cache, torch.bfloat16, "k_cache", 4)
    _need(v_cache, torch.bfloat16, "v_cache", 4)
    _need(slot_pos, torch.int32, "slot_pos", 3)
    _need(slot_score, torch.float32, "slot_score", 3)
    _need(k_new, torch.bfloat16, "k_new", 3)
    _need(v_new, torch.bfloat16, "v_new", 3)
    _need(state, torch.float32, "state", 3)
    B, Hq, D = q.shape
    Hkv, budget = k_cache.shape[1], k_cache.shape[2]
    w = _mlstm_weights(params)
    d = dims(B, Hq, Hkv, budget, D, scale)
    o = out if out is not None else torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    lse = out_lse if out_lse is not None else (
        torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None)
    nbytes = workspace_bytes(OP_DECODE, d)
    ws = workspace if workspace is not None else (
        torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None)
    st = lib().kvpop_decode_step_mlstm(ctypes.byref(d), int(n_sink), int(window), int(pos_q),
                                       _p(k_new), _p(v_new), ctypes.byref(w), _p(state),
                                       _p(k_cache), _p(v_cache), _p(slot_pos), _p(slot_score),
                                       _p(q), _p(o), 1 if o.dtype == torch.bfloat16 else 0, _p(lse),
                                       _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                       _stream())
    _check("kvpop_decode_step_mlstm", st)
    return o, lse


def fwd_lse_sparse(q, k, keep_until, budget=0, scale=0.0, out=None, workspace=None, v=None,
                   out_o=None, out_dtype=torch.float32):
    """Sparse causal log-normalizers LSE [B,Hq,S] fp32 over the running
    top-k mask (App. D.3, C.1): key t counts for row d while
    t <= d < keep_until[t].  ``budget`` is the budget keep_until was made
    with: each block of queries then attends over its listed keys only
    (0: every causal key is read and tested).  With v, also the sparse
    attention output O [B,Hq,S,D] (App. I), returned as (lse, o); every
    causal key is then read and tested."""
    _need(q, torch.bfloat16, "q", 4)
    _need(k, torch.bfloat16, "k", 4)
    _need(keep_until, torch.int32, "keep_until", 3)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, S, D) or tuple(keep_until.shape) != (B, Hkv, S):
        raise ValueError("k / keep_until shape mismatch")
    lse = out if out is not None else torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _need(lse, torch.float32, "lse")
    o = _attn_out(q, v, k, out_o, out_dtype)
    d = dims(B, Hq, Hkv, S, D, scale)
    nbytes = (workspace_bytes(OP_FWD_ATTN, d) if v is not None
              else workspace_bytes(OP_FWD_LSE_SPARSE, d, budget))
    ws = workspace if workspace is not None else (
        torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None)
    st = lib().kvpop_fwd_lse_sparse(ctypes.byref(d), _p(q), _p(k), _p(v), _p(keep_until),
                                    int(budget), _p(lse), _p(o),
                                    1 if o is not None and o.dtype == torch.bfloat16 else 0,
                                    _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream())
    _check("kvpop_fwd_lse_sparse", st)
    return lse if o is None else (lse, o)


def future_attn_target(q, k, lse, window, lookahead=-1, agg="sum", count_normalize=False,
                       per_qhead=False, scale=0.0, out=None, workspace=None):
    """Future-attention mass [B,Hkv,S] (and per-query-head [B,Hq,S]) (App. D.2, B.1-B.2)."""
    _need(q, torch.bfloat16, "q", 4)
    _need(k, torch.bfloat16, "k", 4)
    _need(lse, torch.float32, "lse", 3)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if tuple(k.shape) != (B, Hkv, S, D) or tuple(lse.shape) != (B, Hq, S):
        raise ValueError("shape mismatch")
    d = dims(B, Hq, Hkv, S, D, scale)
    mass = out if out is not None else torch.empty((B, Hkv, S), dtype=torch.float32, device=q.device)
    ph = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if per_qhead else None
    nbytes = workspace_bytes(OP_FUTURE_TARGET, d, window)
    ws = workspace if workspace is not None else torch.empty(max(nbytes, 256), dtype=torch.uint8,
                                                             device=q.device)
    st = lib().kvpop_future_attn_target(ctypes.byref(d), _p(q), _p(k), _p(lse), int(window),
                                        int(lookahead), AGG[agg], int(bool(count_normalize)),
                                        _p(mass), _p(ph), _p(ws), ws.numel() * ws.element_size(),
                                        _stream())
    _check("kvpop_future_attn_target", st)
    return (mass, ph) if per_qhead else mass


def evict_select(scores, n_sink, window, budget, k=None, v=None, want_score=True,
                 out_pos=None, out_score=None, out_k=None, out_v=None):
    """Retention (Sec. 3, App. C.1): slot_pos [B,Hkv,budget] int32, slot_score, and the
    compacted bf16 caches when k, v are given."""
    _need(scores, torch.float32, "scores", 3)
    B, Hkv, S = scores.shape
    dev = scores.device
    D = 0
    if k is not None:
        _need(k, torch.bfloat16, "k", 4)
        _need(v, torch.bfloat16, "v", 4)
        D = k.shape[-1]
    sp = out_pos if out_pos is not None else torch.empty((B, Hkv, budget), dtype=torch.int32, device=dev)
    ss = out_score if out_score is not None else (
        torch.empty((B, Hkv, budget), dtype=torch.float32, device=dev) if want_score else None)
    kc = vc = None
    if k is not None:
        kc = out_k if out_k is not None else torch.empty((B, Hkv, budget, D), dtype=torch.bfloat16, device=dev)
        vc = out_v if out_v is not None else torch.empty((B, Hkv, budget, D), dtype=torch.bfloat16, device=dev)
    st = lib().kvpop_evict_select(B, Hkv, S, D, int(n_sink), int(window), int(budget), _p(scores),
                                  _p(k), _p(v), _p(sp), _p(ss), _p(kc), _p(vc), _stream())
    _check("kvpop_evict_select", st)
    return sp, ss, kc, vc


def decode_attend(q, k_cache, v_cache, slot_pos, out_dtype=torch.float32, want_lse=True,
                  scale=0.0, out=None, out_lse=None, workspace=None):
    """Decode attention over the bounded cache (Sec. 3, App. C.1): o [B,Hq,D], lse [B,Hq]."""
    _need(q, torch.bfloat16, "q", 3)
    _need(k_cache, torch.bfloat16, "k_cache", 4)
    _need(v_cache, torch.bfloat16, "v_cache", 4)
    _need(slot_pos, torch.int32, "slot_pos", 3)
    B, Hq, D = q.shape
    Hkv, n = k_cache.shape[1], k_cache.shape[2]
    d = dims(B, Hq, Hkv, n, D, scale)
    o = out if out is not None else torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    lse = out_lse if out_lse is not None else (
        torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None)
    nbytes = workspace_bytes(OP_DECODE, d)
    ws = workspace if workspace is not None else (
        torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None)
    st = lib().kvpop_decode_attend(ctypes.byref(d), _p(q), _p(k_cache), _p(v_cache), _p(slot_pos),
                                   _p(o), 1 if o.dtype == torch.bfloat16 else 0, _p(lse), _p(ws),
                                   0 if ws is None else ws.numel(), _stream())
    _check("kvpop_decode_attend", st)
    return o, lse


def decode_attend_noalloc(q, k_cache, v_cache, slot_pos, out_dtype=torch.float32, want_lse=True,
                          scale=0.0, out=None, out_lse=None):
    """decode_attend through kvpop_decode_attend_noalloc: no workspace, the
    library's fixed device array holds the split partials (for callers that
    cannot allocate; the outputs are still the caller's)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(k_cache, torch.bfloat16, "k_cache", 4)
    _need(v_cache, torch.bfloat16, "v_cache", 4)
    _need(slot_pos, torch.int32, "slot_pos", 3)
    B, Hq, D = q.shape
    Hkv, n = k_cache.shape[1], k_cache.shape[2]
    d = dims(B, Hq, Hkv, n, D, scale)
    o = out if out is not None else torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    lse = out_lse if out_lse is not None else (
        torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None)
    st = lib().kvpop_decode_attend_noalloc(ctypes.byref(d), _p(q), _p(k_cache), _p(v_cache),
                                           _p(slot_pos), _p(o),
                                           1 if o.dtype == torch.bfloat16 else 0, _p(lse),
                                           _stream())
    _check("kvpop_decode_attend_noalloc", st)
    return o, lse


def score_mlp(keys, w1, b1, w2, b2, out=None):
    """Headwise MLP scores of keys [B,Hkv,n,D] -> [B,Hkv,n] fp32 (App. E.2)."""
    _need(keys, torch.bfloat16, "keys", 4)
    for t, n in ((w1, "w1"), (b1, "b1"), (w2, "w2"), (b2, "b2")):
        _need(t, torch.float32, n)
    B, Hkv, n, D = keys.shape
    hidden = w1.shape[1]
    sc = out if out is not None else torch.empty((B, Hkv, n), dtype=torch.float32, device=keys.device)
    st = lib().kvpop_score_mlp(B, Hkv, n, D, hidden, _p(keys), _p(w1), _p(b1), _p(w2), _p(b2),
                               _p(sc), _stream())
    _check("kvpop_score_mlp", st)
    return sc


def cache_step(k_cache, v_cache, slot_pos, slot_score, k_new, v_new, pos_q, n_sink, window,
               delay, mlp=None, scores_r=None):
    """One bounded-cache decode step in place (Sec. 3, App. C.1, App. E.4).

    mlp: (w1, b1, w2, b2) to score token pos_q - delay from its cached key, or
    scores_r [B,Hkv] fp32 to supply that score directly.
    """
    _need(k_cache, torch.bfloat16, "k_cache", 4)
    _need(v_cache, torch.bfloat16, "v_cache", 4)
    _need(slot_pos, torch.int32, "slot_pos", 3)
    _need(slot_score, torch.float32, "slot_score", 3)
    _need(k_new, torch.bfloat16, "k_new", 3)
    _need(v_new, torch.bfloat16, "v_new", 3)
    B, Hkv, budget, D = k_cache.shape
    w1 = b1 = w2 = b2 = None
    hidden = 0
    if mlp is not None:
        w1, b1, w2, b2 = mlp
        hidden = w1.shape[1]
    if scores_r is not None:
        _need(scores_r, torch.float32, "scores_r")
    st = lib().kvpop_cache_step(B, Hkv, D, int(n_sink), int(window), budget, int(delay), int(pos_q),
                                _p(k_new), _p(v_new), _p(w1), _p(b1), _p(w2), _p(b2), hidden,
                                _p(scores_r), _p(k_cache), _p(v_cache), _p(slot_pos),
                                _p(slot_score), _stream())
    _check("kvpop_cache_step", st)


def decode_step(q, k_cache, v_cache, slot_pos, slot_score, k_new, v_new, pos_q, n_sink, window,
                delay, mlp=None, scores_r=None, out_dtype=torch.float32, want_lse=True, scale=0.0,
                out=None, out_lse=None, workspace=None):
    """One bounded-cache decode step in place, then decode attention over the
    updated cache (Sec. 3, App. C.1, App. E.4): o [B,Hq,D], lse [B,Hq].
    Same effect as cache_step(...) followed by decode_attend(...)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(k_cache, torch.bfloat16, "k_cache", 4)
    _need(v_cache, torch.bfloat16, "v_cache", 4)
    _need(slot_pos, torch.int32, "slot_pos", 3)
    _need(slot_score, torch.float32, "slot_score", 3)
    _need(k_new, torch.bfloat16, "k_new", 3)
    _need(v_new, torch.bfloat16, "v_new", 3)
    B, Hq, D = q.shape
    Hkv, budget = k_cache.shape[1], k_cache.shape[2]
    w1 = b1 = w2 = b2 = None
    hidden = 0
    if mlp is not None:
        w1, b1, w2, b2 = mlp
        hidden = w1.shape[1]
    if scores_r is not None:
        _need(scores_r, torch.float32, "scores_r")
    d = dims(B, Hq, Hkv, budget, D, scale)
    o = out if out is not None else torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    lse = out_lse if out_lse is not None else (
        torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None)
    nbytes = workspace_bytes(OP_DECODE, d)
    ws = workspace if workspace is not None else (
        torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None)
    st = lib().kvpop_decode_step(ctypes.byref(d), int(n_sink), int(window), int(delay), int(pos_q),
                                 _p(k_new), _p(v_new), _p(w1), _p(b1), _p(w2), _p(b2), hidden,
                                 _p(scores_r), _p(k_cache), _p(v_cache), _p(slot_pos),
                                 _p(slot_score), _p(q), _p(o), 1 if o.dtype == torch.bfloat16 else 0,
                                 _p(lse), _p(ws), 0 if ws is None else ws.numel(), _stream())
    _check("kvpop_decode_step", st)
    return o, lse
