"""Dense brute force for tiny sizes -- TEST INFRASTRUCTURE ONLY.

This materialises the full S x S score and probability matrices in float64
with numpy and reads every quantity off them with masks.  It is a second
route to the same definitions as ``kvpop_oracle.c`` (which never forms the
matrix), used to pin the oracle before it is trusted.

App. D.1 of the KVpop summary states that the future-attention target is
exactly the per-key log-sum-exp over future queries of the dense softmax,
so column sums of the masked dense probability matrix are the definition.
"""
import math

import numpy as np
from scipy.special import logsumexp


def repeat_kv(k, G):
    """KV head h serves query heads h*G .. h*G+G-1 (grouped-query sharing)."""
    return np.repeat(np.asarray(k, np.float64), G, axis=1)


def scores(q, k, scale=None):
    q = np.asarray(q, np.float64)
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    kk = repeat_kv(k, G)
    return sc * np.matmul(q, np.swapaxes(kk, -1, -2))  # [B,Hq,S(d),S(t)]


def causal_mask(S):
    return np.tril(np.ones((S, S), dtype=bool))


def lse(q, k, scale=None):
    z = scores(q, k, scale)
    S = z.shape[-1]
    zm = np.where(causal_mask(S), z, -np.inf)
    return logsumexp(zm, axis=-1)


def probs(q, k, scale=None):
    z = scores(q, k, scale)
    S = z.shape[-1]
    ls = lse(q, k, scale)
    p = np.exp(z - ls[..., None])
    return np.where(causal_mask(S), p, 0.0)


def future_mask(S, window, lookahead=-1):
    """mask[d, t] = True where query d counts toward key t: t+w <= d (<= t+w+L)."""
    d = np.arange(S)[:, None]
    t = np.arange(S)[None, :]
    m = d >= t + window
    if lookahead >= 0:
        m &= d <= t + window + lookahead
    return m


def mass_per_head(q, k, window, lookahead=-1, scale=None):
    """m[b, g, t] = column sums of the masked dense probability matrix."""
    p = probs(q, k, scale)
    S = p.shape[-1]
    return np.where(future_mask(S, window, lookahead), p, 0.0).sum(axis=-2)


def aggregate(m, Hkv, agg):
    B, Hq, S = m.shape
    G = Hq // Hkv
    mg = m.reshape(B, Hkv, G, S)
    if agg == "sum":
        return mg.sum(axis=2)
    if agg == "mean":
        return mg.mean(axis=2)
    if agg == "max":
        return mg.max(axis=2)
    raise ValueError(agg)


def count(S, window, lookahead=-1):
    t = np.arange(S)
    n = np.clip(S - t - window, 0, None)
    if lookahead >= 0:
        n = np.minimum(n, lookahead + 1)
    return n


def select_positions(scores_row, n_sink, window, budget):
    """Retained position set of one row, by a textbook sort (Python's sorted).

    Order: finite/inf scores before NaN, higher score first, lower position
    first on ties (Python compares -0.0 == 0.0).
    """
    S = len(scores_row)
    k = budget - n_sink - window
    elig = list(range(n_sink, max(n_sink, S - window)))

    def key(t):
        s = float(scores_row[t])
        return (math.isnan(s), 0.0 if math.isnan(s) else -s, t)

    chosen = sorted(elig, key=key)[:max(k, 0)]
    sinks = list(range(min(n_sink, S)))
    win = list(range(max(S - window, n_sink), S))
    return sorted(set(sinks) | set(chosen) | set(win)), sorted(chosen)


def decode(q, kc, vc, slot_pos, scale=None):
    """Softmax attention of q [B,Hq,D] over valid slots, float64."""
    q = np.asarray(q, np.float64)
    B, Hq, D = q.shape
    Hkv = kc.shape[1]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    o = np.zeros((B, Hq, D))
    ls = np.full((B, Hq), -np.inf)
    for b in range(B):
        for g in range(Hq):
            h = g // G
            valid = slot_pos[b, h] >= 0
            if not valid.any():
                continue
            K = np.asarray(kc[b, h][valid], np.float64)
            V = np.asarray(vc[b, h][valid], np.float64)
            z = sc * K @ q[b, g]
            ls[b, g] = logsumexp(z)
            o[b, g] = np.exp(z - ls[b, g]) @ V
    return o, ls
