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


def priorities(scores_row, log_decay=0.0):
    """Static priorities pi_t = sigma_t + lambda * t, each operation rounded
    to float32 (numpy float32 scalars round after every operation)."""
    lam = np.float32(log_decay)
    return [np.float32(np.float32(scores_row[t]) + np.float32(lam * np.float32(t)))
            for t in range(len(scores_row))]


def running_sets(scores_row, n_sink, window, budget, log_decay=0.0):
    """Per query d, the retained set R_d and the cutoff token of one row, by
    sorting the pool P_d = [s, d - w] afresh at every d (Python's sorted).
    Returns (list of sets R_d, list of cutoff tokens or -1)."""
    S = len(scores_row)
    k = budget - n_sink - window
    pi = priorities(scores_row, log_decay)

    def key(t):
        s = float(pi[t])
        return (math.isnan(s), 0.0 if math.isnan(s) else -s, t)

    R, cut = [], []
    for d in range(S):
        pool = list(range(n_sink, d - window + 1))
        chosen = sorted(pool, key=key)[:max(k, 0)]
        sinks = set(range(min(n_sink, d + 1)))
        win = set(range(max(d - window + 1, 0), d + 1))
        R.append(sinks | win | set(chosen))
        cut.append(chosen[-1] if k > 0 and len(pool) >= k else -1)
    return R, cut


def keep_until_from_sets(R, S):
    """First query d >= t with t not in R_d (S if none), for every t."""
    out = []
    for t in range(S):
        d = t
        while d < S and t in R[d]:
            d += 1
        out.append(d)
    return out


def lse_masked(q, k, member, scale=None):
    """LSE over an explicit membership mask member[b, h, d, t] (bool)."""
    z = scores(q, k, scale)
    G = z.shape[1] // member.shape[1]
    m = np.repeat(member, G, axis=1)
    return logsumexp(np.where(m, z, -np.inf), axis=-1)


def attn_masked(q, k, v, member, scale=None):
    """Softmax attention output over an explicit membership mask
    member[b, h, d, t] (bool), float64: the probability matrix of the
    masked rows times V.  Returns (o [B,Hq,S,D], lse [B,Hq,S])."""
    z = scores(q, k, scale)
    G = z.shape[1] // member.shape[1]
    m = np.repeat(member, G, axis=1)
    zm = np.where(m, z, -np.inf)
    ls = logsumexp(zm, axis=-1)
    p = np.where(m, np.exp(zm - ls[..., None]), 0.0)
    return np.matmul(p, repeat_kv(v, G)), ls


def mlstm_scores_unstabilised(keys, values, params, window):
    """The delayed mLSTM scores from the unstabilised recurrence, float64:
    C_q = sum_{t<=q} (prod_{j=t+1..q} sigmoid(f_j)) exp(i_t) val_t phi_t^T (same
    for n), h = C_q r / max(|n_q . r|, 1), sigma = wo . silu(h) + bo.  The
    stabiliser m scales C and n by exp(-m) and the floor by the same factor,
    so both forms give the same h."""
    k = np.asarray(keys, np.float64)
    v = np.asarray(values, np.float64)
    B, H, n, D = k.shape
    pr = {name: np.asarray(val, np.float64) for name, val in params.items()}

    def hh(z):
        a = np.exp(z - z.max())
        b = np.exp(-z - (-z).max())
        return np.concatenate([a / a.sum(), b / b.sum()])

    out = np.full((B, H, n), np.nan)
    for b in range(B):
        for h in range(H):
            x = np.concatenate([k[b, h], v[b, h]], axis=-1)  # [n, 2D]
            ig = x @ pr["wi"][h] + pr["bi"][h]
            fg = x @ pr["wf"][h] + pr["bf"][h]
            sf = 1.0 / (1.0 + np.exp(-fg))
            phi = np.stack([hh(pr["wk"][h] @ x[t]) for t in range(n)])
            val = x @ pr["wv"][h].T
            for q in range(window, n):
                u = q - window
                decay = np.array([np.prod(sf[t + 1:q + 1]) for t in range(q + 1)])
                wgt = decay * np.exp(ig[:q + 1])
                C = (val[:q + 1] * wgt[:, None]).T @ phi[:q + 1]
                nr = (phi[:q + 1] * wgt[:, None]).sum(0)
                r = hh(pr["wr"][h] @ x[u])
                hv = C @ r / max(abs(nr @ r), 1.0)
                out[b, h, u] = pr["wo"][h] @ (hv / (1.0 + np.exp(-hv))) + pr["bo"][h]
    return out
