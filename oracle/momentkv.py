"""MomentKV variant, fp64 reference -- TEST INFRASTRUCTURE ONLY (see oracle/__init__).

Per (sequence, KV head) moment statistics of the evicted set [MKV part 1]: the count
n_e, the key sum s_k, the value sum s_v and the outer-product sum S = sum v k^T.
They give the first-order estimate of the evicted attention output [MKV part 2],
the residual-based eviction score [MKV part 3] and the mixing weight from the
Jensen lower bound of the evicted partition function [MKV part 4].
"""
import math

import numpy as np

from . import indexmem as im


# ----------------------------------------------------------------------------- moments

def empty(d):
    return dict(n=0, sk=np.zeros(d), sv=np.zeros(d), S=np.zeros((d, d)))


def add(mom, K_rows, V_rows):
    """Fold evicted rows into the four running sums [MKV part 1]."""
    K_rows = np.asarray(K_rows, np.float64).reshape(-1, mom["sk"].shape[0])
    V_rows = np.asarray(V_rows, np.float64).reshape(-1, mom["sv"].shape[0])
    return dict(n=mom["n"] + K_rows.shape[0], sk=mom["sk"] + K_rows.sum(0),
                sv=mom["sv"] + V_rows.sum(0), S=mom["S"] + V_rows.T @ K_rows)


def stats(mom):
    """Key mean, value mean and the (unnormalised) value-key covariance
    S~ = sum (v - v_bar)(k - k_bar)^T = S - s_v s_k^T / n_e  [MKV part 1].
    Reading: S~ is unnormalised, the only form for which the part-2 equation is the
    first-order expansion of softmax about k_bar."""
    n = mom["n"]
    kbar = mom["sk"] / n
    vbar = mom["sv"] / n
    St = mom["S"] - np.outer(mom["sv"], mom["sk"]) / n
    return kbar, vbar, St


# ----------------------------------------------------------------------------- V1

def alpha(Qwin, K, q_pos, scale, G):
    """Reading of the attention weight alpha_j [MKV part 3]: the causal softmax weight
    of key j averaged over the window's queries and the G query heads of the KV group.
    Qwin [W, H_q, d], K [L, H_kv, d] -> alpha [H_kv, L]."""
    Qwin = np.asarray(Qwin, np.float64)
    K = np.asarray(K, np.float64)
    W, H_q, d = Qwin.shape
    L, H_kv, _ = K.shape
    out = np.zeros((H_kv, L))
    for g in range(H_kv):
        for s in range(W):
            n = int(q_pos[s]) + 1
            for h in range(g * G, (g + 1) * G):
                logit = K[:n, g, :] @ Qwin[s, h] * scale
                w = np.exp(logit - logit.max())
                out[g, :n] += w / w.sum()
    return out / (W * G)


def residual(k, v, mom, d):
    """Moment residual r_j = v_j - v_bar - S~ k_j / (n_e sqrt d) [MKV part 3, equation];
    with nothing evicted yet (n_e = 0) the residual is v_j itself."""
    v = np.asarray(v, np.float64)
    if mom["n"] == 0:
        return v.copy()
    _, vbar, St = stats(mom)
    return v - vbar - (np.asarray(k, np.float64) @ St.T) / (mom["n"] * math.sqrt(d))


def score(alpha_j, k, v, mom, d):
    """Eviction score alpha_j * ||r_j|| [MKV part 3, equation].  k, v [n, d]."""
    return np.asarray(alpha_j, np.float64) * np.linalg.norm(residual(k, v, mom, d), axis=-1)


def select_round(scores, pos, keep):
    """Keep the `keep` highest scores (ties keep the lower position); returns the kept
    and the evicted indices into `pos`, each in ascending position order."""
    order = sorted(range(len(pos)), key=lambda j: (-im.select_key(scores[j]), int(pos[j])))
    kept = sorted(order[:keep], key=lambda j: pos[j])
    ev = sorted(order[keep:], key=lambda j: pos[j])
    return kept, ev


def n_rounds(L, B):
    r, cur = 0, L
    while cur > B:
        cur = max(B, -(-cur // 2))
        r += 1
    return r


def prefill(Qwin, K, V, B, q_pos=None):
    """Moment-informed eviction of one sequence, per KV head.

    Reading: alpha is computed once; eviction runs in rounds, each keeping
    max(B, ceil(n/2)) of the n currently retained tokens by score, so the retained
    count halves until it reaches B; each round scores with the moments accumulated so
    far, then folds its evicted tokens in.  Returns per-head kept positions, moments
    and the per-round selections.
    """
    Qwin = np.asarray(Qwin, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    W, H_q, d = Qwin.shape
    L, H_kv, _ = K.shape
    G = H_q // H_kv
    if q_pos is None:
        q_pos = np.arange(L - W, L)
    scale = 1.0 / math.sqrt(d)
    al = alpha(Qwin, K, q_pos, scale, G)
    heads = []
    for g in range(H_kv):
        pos = np.arange(L)
        mom = empty(d)
        rounds = []
        while len(pos) > B:
            keep = max(B, -(-len(pos) // 2))
            sc = score(al[g, pos], K[pos, g], V[pos, g], mom, d)
            kept, ev = select_round(sc, pos, keep)
            rounds.append(dict(pos=pos.copy(), scores=sc, kept=pos[kept], evicted=pos[ev]))
            mom = add(mom, K[pos[ev], g], V[pos[ev], g])
            pos = pos[kept]
        heads.append(dict(kept=pos, mom=mom, rounds=rounds))
    return dict(alpha=al, heads=heads)


# ----------------------------------------------------------------------------- V3

def evicted_estimate(q, mom, d):
    """First-order estimate f^_E(q) = v_bar + S~ q / (n_e sqrt d) [MKV part 2, equation]."""
    _, vbar, St = stats(mom)
    return vbar + St @ np.asarray(q, np.float64) / (mom["n"] * math.sqrt(d))


def log_Z_hat(q, mom, d):
    """Jensen lower bound of the evicted partition function [MKV part 4]:
    Z_E = sum_i exp(q.k_i/sqrt d) >= n_e exp(q.k_bar/sqrt d) = Z^_E; returns log Z^_E."""
    kbar = mom["sk"] / mom["n"]
    return math.log(mom["n"]) + float(np.asarray(q, np.float64) @ kbar) / math.sqrt(d)


def mix(q, f_R, lse_R, mom, d):
    """Normalization-corrected output f^ = w_R f_R + (1 - w_R) f^_E [MKV part 4, equation]
    with w_R = Z_R / (Z_R + Z^_E) = sigmoid(lse_R - log Z^_E); n_e = 0 gives f_R."""
    if mom["n"] == 0:
        return np.asarray(f_R, np.float64).copy(), 1.0
    w = float(im.sigmoid(lse_R - log_Z_hat(q, mom, d)))
    return w * np.asarray(f_R, np.float64) + (1.0 - w) * evicted_estimate(q, mom, d), w


def decode(q_steps, k_steps, v_steps, K, V, heads, T=None):
    """Decode over each KV head's retained tokens with the NC mix.  Reading: each step
    appends the new K/V before attending; no eviction during decode.
    q_steps [T, H_q, d], k/v_steps [T, H_kv, d]; K, V the prefill [L, H_kv, d].
    Returns f^ [T, H_q, d], lse_R [T, H_q] and w_R [T, H_q]."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    T = q_steps.shape[0] if T is None else T
    H_q, d = q_steps.shape[1], q_steps.shape[2]
    H_kv = K.shape[1]
    G = H_q // H_kv
    scale = 1.0 / math.sqrt(d)
    Kr = [K[heads[g]["kept"], g] for g in range(H_kv)]
    Vr = [V[heads[g]["kept"], g] for g in range(H_kv)]
    out = np.zeros((T, H_q, d))
    lses = np.zeros((T, H_q))
    ws = np.zeros((T, H_q))
    for t in range(T):
        for g in range(H_kv):
            Kr[g] = np.vstack([Kr[g], np.asarray(k_steps[t, g], np.float64)[None]])
            Vr[g] = np.vstack([Vr[g], np.asarray(v_steps[t, g], np.float64)[None]])
        for h in range(H_q):
            g = h // G
            q = np.asarray(q_steps[t, h], np.float64)
            f_R, lse_R = im.attention_state(q, Kr[g], Vr[g], scale)
            out[t, h], ws[t, h] = mix(q, f_R, lse_R, heads[g]["mom"], d)
            lses[t, h] = lse_R
    return out, lses, ws
