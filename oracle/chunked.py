"""Chunked pre-eviction during prefill, fp64 reference -- TEST INFRASTRUCTURE ONLY.

[IM 2.A, pre-eviction]: the indexer predicts which entries to keep before the full prefill
computation, saving memory.  Here the prefill's tokens arrive in chunks and the retained
set returns to the budget after each chunk, so at most B + C tokens are ever held.

Reading (the pages give no chunk schedule):
  - the L prefill tokens arrive in chunks of C (the last one may be shorter; every chunk
    holds at least W and R tokens);
  - after the chunk that ends at position e, the indexer window is its last W positions
    e-W .. e-1 (their hidden states and model queries);
  - each window query scores every pooled key and every key of the chunk at or before it;
    a pooled key's importance becomes the running max of its importance and these
    scores, a chunk key's importance is its max over this window;
  - the budget selection of the one-shot prefill (the recent R positions, here the
    chunk's last R, plus the top B - R of the rest, ties keeping the lower position) runs
    over pool and chunk together, in position order;
  - the evicted tokens are folded into M, b in ascending position order, one decayed fold
    per chunk;
  - one chunk covering the whole prefill is the one-shot pre-eviction.
"""
import numpy as np

from . import indexmem as im


def prefill_chunked(X, Q, K, V, W_kI, gamma_k, W_qI, gamma_q, W_g, B, R, lam, C, W,
                    recent_inclusive=True, act="relu", eps=1e-6):
    """One sequence of one layer.  X [L, D], Q [L, H_q, d] (model queries; only each chunk's
    last W rows are read), K, V [L, H_kv, d], all float64.  Returns the final pool
    (positions ascending, importances, indexer keys, K, V rows [n, H_kv, d]), M, b and per
    chunk the pooled positions, the evicted positions and the importances over pool and
    chunk before the selection."""
    X = np.asarray(X, np.float64)
    L, H_kv, d = K.shape
    d_I = np.asarray(W_kI).shape[0]
    pos = np.zeros(0, np.int64)
    khat = np.zeros((0, d_I))
    I = np.zeros(0)
    Kp = np.zeros((0, H_kv, d))
    Vp = np.zeros((0, H_kv, d))
    M = np.zeros((H_kv, d, d))
    b = np.zeros((H_kv, d))
    steps = []
    for s in range(0, L, C):
        e = min(L, s + C)
        assert e - s >= W and e - s >= R, "every chunk holds the window and the recent tokens"
        kh_c = im.indexer_keys(X[s:e], W_kI, gamma_k, eps)
        q_hat, gate = im.indexer_queries(Q[e - W:e], X[e - W:e], W_qI, gamma_q, W_g, eps)
        n_pool = len(pos)
        vpos = np.concatenate([pos, np.arange(s, e)])
        vk = np.vstack([khat, kh_c])
        # pool and chunk in position order: window query at position e - W + i sits at
        # index n_pool + (e - W - s) + i and sees every key up to it
        q_idx = n_pool + (e - W - s) + np.arange(W)
        I_cur = im.importance(im.score_matrix(q_hat, gate, vk, q_idx, act))
        Iv = np.concatenate([np.maximum(I, I_cur[:n_pool]), I_cur[n_pool:]])
        idx, slot_map = im.topk_select(Iv, B, R, recent_inclusive)
        ev = im.evicted_in_order(slot_map)
        Kv = np.concatenate([Kp, np.asarray(K[s:e], np.float64)])
        Vv = np.concatenate([Vp, np.asarray(V[s:e], np.float64)])
        for g in range(H_kv):
            M[g], b[g] = im.memory_build(Kv[ev, g], Vv[ev, g], lam, M[g], b[g])
        steps.append(dict(I=Iv.copy(), vpos=vpos.copy(), kept=vpos[idx], evicted=vpos[ev]))
        pos, khat, I, Kp, Vp = vpos[idx], vk[idx], Iv[idx], Kv[idx], Vv[idx]
    return dict(pos=pos, I=I, k_hat=khat, K=Kp, V=Vp, M=M, b=b, steps=steps)
