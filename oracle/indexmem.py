"""IndexMem hot path, fp64 reference -- TEST INFRASTRUCTURE ONLY (see oracle/__init__).

Steps, in the pages' order: indexer keys and queries, dense score matrix A and its
per-key max-pool I, pre-eviction top-k, K/V compaction, latent-memory build, decode
attention over the retained cache with (a, Z) states, and the residual readout.
All arithmetic is float64; storage-format inputs (bf16 bit patterns or fp32) are
decoded exactly first.
"""
import numpy as np


# ----------------------------------------------------------------------------- formats

def f64(a, dtype: str) -> np.ndarray:
    """Exact decode of a storage-format array: bf16 bit patterns (uint16) or fp32."""
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------- elementwise

def phi(x):
    """phi = elu + 1: x + 1 for x > 0 and exp(x) for x <= 0 (this library's fixed choice
    for the feature map of the memory readout; the pages name M, b and g(q) only)."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, 1.0 / (1.0 + np.exp(-np.abs(x))),
                    np.exp(-np.abs(x)) / (1.0 + np.exp(-np.abs(x))))


def rmsnorm(x, gamma, eps):
    """RMS normalisation over the last axis with learnable scale gamma.
    Reading: the indexer's "QK norm" [IM 2.A] is RMSNorm over d_I."""
    x = np.asarray(x, dtype=np.float64)
    return np.asarray(gamma, np.float64) * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


# ----------------------------------------------------------------------------- A1, A2

def indexer_keys(X, W_kI, gamma_k, eps=1e-6):
    """One shared indexer key per token, projected from the hidden state and QK-normed
    [IM 2.A, architecture].  X [L, D], W_kI [d_I, D] -> k_hat [L, d_I]."""
    return rmsnorm(np.asarray(X, np.float64) @ np.asarray(W_kI, np.float64).T, gamma_k, eps)


def indexer_head_map(H_I, H_q):
    """Reading: indexer head h down-projects model query head floor(h * H_q / H_I)."""
    return [(h * H_q) // H_I for h in range(H_I)]


def indexer_queries(Qwin, Xwin, W_qI, gamma_q, W_g, eps=1e-6):
    """Down-projected, QK-normed multi-head indexer queries and their gates [IM 2.A].

    Qwin [W, H_q, d] model queries, Xwin [W, D] hidden states of the same positions,
    W_qI [H_I, d_I, d], W_g [H_I, D].  Returns q_hat [W, H_I, d_I] and gate [W, H_I].
    Reading: the learnable gate is g[s, h] = sigmoid(W_g[h] . x_s), one scalar per query
    position and indexer head, so every head contribution is weighted by a value in (0, 1).
    """
    Qwin = np.asarray(Qwin, np.float64)
    W_qI = np.asarray(W_qI, np.float64)
    H_I = W_qI.shape[0]
    c = indexer_head_map(H_I, Qwin.shape[1])
    qI = np.stack([Qwin[:, c[h], :] @ W_qI[h].T for h in range(H_I)], axis=1)
    q_hat = rmsnorm(qI, gamma_q, eps)
    gate = sigmoid(np.asarray(Xwin, np.float64) @ np.asarray(W_g, np.float64).T)
    return q_hat, gate


# ----------------------------------------------------------------------------- A3

def score_matrix(q_hat, gate, k_hat, q_pos, act="relu"):
    """Dense query-to-key score matrix A [IM 2.A, function]: A[s, t] is the importance of
    key t for window query s.

    A[s, t] = sum_h gate[s, h] * act(q_hat[s, h] . k_hat[t] / sqrt(d_I))   for t <= q_pos[s]
    and -inf for t > q_pos[s] (a query never scores a later token).
    Reading: act is a per-head ReLU (act="none" gives the linear form); the logit scale
    is 1/sqrt(d_I).  Returns A [W, L].
    """
    q_hat = np.asarray(q_hat, np.float64)
    k_hat = np.asarray(k_hat, np.float64)
    d_I = k_hat.shape[1]
    logits = np.einsum("shi,ti->sht", q_hat, k_hat) / np.sqrt(d_I)   # [W, H_I, L]
    if act == "relu":
        logits = np.maximum(logits, 0.0)
    elif act != "none":
        raise ValueError(act)
    A = np.einsum("sh,sht->st", np.asarray(gate, np.float64), logits)
    L = k_hat.shape[0]
    causal = np.arange(L)[None, :] > np.asarray(q_pos)[:, None]
    return np.where(causal, -np.inf, A)


def importance(A):
    """Per-key importance: the max-pool of A over the observation window's queries
    [IM 2.A, training: running-max aggregation].  I[t] = max_s A[s, t]."""
    return np.max(A, axis=0)


def importance_streaming(q_hat, gate, k_hat, q_pos, act="relu"):
    """The same I computed as a running max, one query at a time, never holding A."""
    L = k_hat.shape[0]
    I = np.full(L, -np.inf)
    for s in range(q_hat.shape[0]):
        row = score_matrix(q_hat[s:s + 1], gate[s:s + 1], k_hat, np.asarray(q_pos)[s:s + 1], act)[0]
        I = np.maximum(I, row)
    return I


# ----------------------------------------------------------------------------- A4

def select_key(score):
    """Ordering key of a score: NaN counts as -inf and -0 as +0."""
    s = float(score)
    if s != s:
        return -np.inf
    return s + 0.0


def topk_select(I, B, R=0, recent_inclusive=True):
    """Pre-eviction [IM 2.A]: pick the retained entries from the indexer scores alone.

    Kept = the last R positions (recent window) plus the highest-scoring n_top of the
    positions before them, ordered by (score descending, position ascending), so ties
    keep the lower position.  n_top = B - R when the recent window counts inside the
    budget, else B.  A budget covering all L positions keeps everything.

    Returns idx (kept positions, ascending) and slot_map [L] int64: slot_map[t] = slot
    of t in the compact cache (its rank among kept positions) if kept, else -i where
    i = 1..n is t's rank among the evicted positions in ascending order.
    """
    I = np.asarray(I)
    L = I.shape[0]
    if recent_inclusive:
        assert R <= B, "budget must cover the recent window"
        n_top = B - R
    else:
        n_top = B
    R = min(R, L)
    n_cand = L - R
    if n_top >= n_cand:
        kept = list(range(L))
    else:
        order = sorted(range(n_cand), key=lambda t: (-select_key(I[t]), t))
        kept = sorted(order[:n_top]) + list(range(n_cand, L))
    keep = np.zeros(L, bool)
    keep[kept] = True
    slot_map = np.zeros(L, np.int64)
    s = e = 0
    for t in range(L):
        if keep[t]:
            slot_map[t] = s
            s += 1
        else:
            e += 1
            slot_map[t] = -e
    return np.array(kept, np.int64), slot_map


# ----------------------------------------------------------------------------- A5

def compact(K, V, slot_map, cap):
    """Gather the kept rows of token-major K, V [L, H_kv, d] into head-major
    Kc, Vc [H_kv, cap, d] at their slots (unused slots stay zero)."""
    K = np.asarray(K)
    V = np.asarray(V)
    L, H, d = K.shape
    Kc = np.zeros((H, cap, d), K.dtype)
    Vc = np.zeros((H, cap, d), V.dtype)
    for t in range(L):
        s = slot_map[t]
        if s >= 0:
            Kc[:, s, :] = K[t]
            Vc[:, s, :] = V[t]
    return Kc, Vc


def evicted_in_order(slot_map):
    """Evicted positions e_1 < ... < e_n (ordered by eviction rank)."""
    sm = np.asarray(slot_map)
    ev = np.nonzero(sm < 0)[0]
    return ev[np.argsort(-sm[ev])]


# ----------------------------------------------------------------------------- A6

def memory_build(K_ev, V_ev, lam, M0=None, b0=None):
    """Latent-memory fast weights from evicted tokens [IM 2.B, mechanism: decayed
    outer-product accumulation into a fixed-size state M and stabiliser b].

    Closed form over evicted rows i = 1..n (in eviction order) of one KV head:
        M = lam^n M0 + sum_i lam^(n-i) v_i phi(k_i)^T,   b = lam^n b0 + sum_i lam^(n-i) phi(k_i).
    K_ev, V_ev [n, d]; returns M [d, d] (rows index v, columns index phi(k)) and b [d].
    Reading: prefill evictions are folded in ascending position order.
    """
    K_ev = np.asarray(K_ev, np.float64)
    V_ev = np.asarray(V_ev, np.float64)
    n, d = K_ev.shape
    w = lam ** (n - np.arange(1, n + 1, dtype=np.float64))
    F = phi(K_ev)
    M = (V_ev * w[:, None]).T @ F
    b = w @ F
    if M0 is not None:
        M = M + lam ** n * np.asarray(M0, np.float64)
    if b0 is not None:
        b = b + lam ** n * np.asarray(b0, np.float64)
    return M, b


def memory_update_sequential(K_rows, V_rows, lam, M0, b0):
    """The online form of the same update: one token at a time, M <- lam M + v phi(k)^T."""
    M = np.array(M0, np.float64)
    b = np.array(b0, np.float64)
    for k, v in zip(np.asarray(K_rows, np.float64), np.asarray(V_rows, np.float64)):
        f = phi(k)
        M = lam * M + np.outer(v, f)
        b = lam * b + f
    return M, b


# ----------------------------------------------------------------------------- A8

def attention_state(q, Kb, Vb, scale):
    """Attention state (a, lse) of one query over one key block [ASM, method]:
    a = sum_j softmax_j(scale q.k_j) v_j and lse = log Z = log sum_j exp(scale q.k_j).
    An empty block has Z = 0: lse = -inf and a = 0."""
    q = np.asarray(q, np.float64)
    Kb = np.asarray(Kb, np.float64)
    Vb = np.asarray(Vb, np.float64)
    if Kb.shape[0] == 0:
        return np.zeros(Vb.shape[1]), -np.inf
    s = Kb @ q * scale
    m = np.max(s)
    e = np.exp(s - m)
    Z = np.sum(e)
    return (e @ Vb) / Z, m + np.log(Z)


def merge_states(states):
    """Online-softmax merge of attention states over disjoint key blocks [ASM, method]:
    lse = log sum_c exp(lse_c) and a = sum_c exp(lse_c - lse) a_c."""
    lses = np.array([l for _, l in states], np.float64)
    if np.all(lses == -np.inf):
        return np.zeros_like(states[0][0]), -np.inf
    m = np.max(lses)
    lse = m + np.log(np.sum(np.exp(lses - m)))
    a = sum(np.exp(l - lse) * ai for ai, l in states)
    return a, lse


def decode_attention(q, Kc, Vc, n, scale):
    """Softmax attention of every query head over the first n retained slots.
    q [H_q, d]; Kc, Vc [H_kv, cap, d]; query head h reads KV head h // (H_q / H_kv).
    Returns o_attn [H_q, d] and lse [H_q]."""
    q = np.asarray(q, np.float64)
    H_q = q.shape[0]
    G = H_q // Kc.shape[0]
    o = np.zeros_like(q)
    lse = np.zeros(H_q)
    for h in range(H_q):
        o[h], lse[h] = attention_state(q[h], Kc[h // G, :n], Vc[h // G, :n], scale)
    return o, lse


# ----------------------------------------------------------------------------- A9

def memory_query(q, W_m):
    """Reading of the slow-weight projection layer [IM 2.B, mechanism: a trained projection
    layer and the gate read from M]: the query that addresses M is W_m q, with one d x d
    matrix per layer shared by every query head; the gate keeps the model's query.
    q [H_q, d], W_m [d, d] -> [H_q, d].  W_m = I gives the read-out without projection."""
    return np.asarray(q, np.float64) @ np.asarray(W_m, np.float64).T


def memory_readout(q, M, b, w_g, eps=1e-6, q_mem=None):
    """Memory read-out and its gate, per query head [IM 2.B].

    m(q) = M phi(q~) / (b . phi(q~) + eps) and g(q) = sigmoid(w_g . q) (this library's fixed
    forms; the pages name M, b and g(q) only), with q~ = q_mem (the projected query, see
    memory_query) if given, else q.  Query head h reads the state of its KV head h // G.
    q, q_mem [H_q, d], M [H_kv, d, d], b [H_kv, d], w_g [H_q, d] -> m [H_q, d], g [H_q].
    """
    q = np.asarray(q, np.float64)
    qm = q if q_mem is None else np.asarray(q_mem, np.float64)
    H_q = q.shape[0]
    G = H_q // M.shape[0]
    m = np.zeros_like(q)
    g = np.zeros(H_q)
    for h in range(H_q):
        f = phi(qm[h])
        m[h] = (M[h // G] @ f) / (b[h // G] @ f + eps)
        g[h] = sigmoid(np.asarray(w_g, np.float64)[h] @ q[h])
    return m, g


def residual_output(o_attn, m, g):
    """o = o_attn + g(q) m(q) [IM 2.B, output]."""
    return o_attn + g[:, None] * m


# ----------------------------------------------------------------------------- pipelines

def prefill(X, Qwin, K, V, W_kI, gamma_k, W_qI, gamma_q, W_g, B, R, lam,
            recent_inclusive=True, act="relu", eps=1e-6, cap=None, M0=None, b0=None):
    """Index -> pre-evict -> compact -> memory build for one sequence of one layer.
    All array inputs are float64 (decoded).  X [L, D], Qwin [W, H_q, d], K, V [L, H_kv, d].
    Returns a dict of every intermediate."""
    L, H_kv, d = K.shape
    W = Qwin.shape[0]
    k_hat = indexer_keys(X, W_kI, gamma_k, eps)
    q_hat, gate = indexer_queries(Qwin, X[L - W:], W_qI, gamma_q, W_g, eps)
    q_pos = np.arange(L - W, L)
    A = score_matrix(q_hat, gate, k_hat, q_pos, act)
    I = importance(A)
    idx, slot_map = topk_select(I, B, R, recent_inclusive)
    cap = len(idx) if cap is None else cap
    Kc, Vc = compact(K, V, slot_map, cap)
    ev = evicted_in_order(slot_map)
    M = np.zeros((H_kv, d, d))
    bv = np.zeros((H_kv, d))
    for g in range(H_kv):
        M[g], bv[g] = memory_build(K[ev, g, :], V[ev, g, :], lam,
                                   None if M0 is None else M0[g], None if b0 is None else b0[g])
    return dict(k_hat=k_hat, q_hat=q_hat, gate=gate, A=A, I=I, idx=idx, slot_map=slot_map,
                Kc=Kc, Vc=Vc, M=M, b=bv, n_evicted=len(ev), n_kept=len(idx))


def decode(q_steps, k_steps, v_steps, Kc, Vc, n0, M, b, w_g, eps=1e-6, use_memory=True):
    """Decode steps over the retained cache.  Reading: each step appends the new token's
    K/V at slot n before attending (the query sees itself); no eviction during decode
    and M, b stay fixed.  q_steps [T, H_q, d], k/v_steps [T, H_kv, d].
    Returns o [T, H_q, d], lse [T, H_q] and the grown caches."""
    Kc = np.array(Kc, np.float64)
    Vc = np.array(Vc, np.float64)
    T, H_q, d = q_steps.shape
    scale = 1.0 / np.sqrt(d)
    outs, lses = [], []
    n = n0
    for t in range(T):
        Kc[:, n] = k_steps[t]
        Vc[:, n] = v_steps[t]
        n += 1
        o, lse = decode_attention(q_steps[t], Kc, Vc, n, scale)
        if use_memory:
            m, g = memory_readout(q_steps[t], M, b, w_g, eps)
            o = residual_output(o, m, g)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses), Kc, Vc
