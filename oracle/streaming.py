"""Streaming eviction during decode, fp64 reference -- TEST INFRASTRUCTURE ONLY.

After pre-eviction to a pool of B + R slots, every decode step evicts one token and
folds it into the latent memory online [IM 2.B, mechanism: evicted tokens update M and
b online during inference with a decayed outer product].

Reading (the pages give no step order): per step, with the new token at position p,
  1. its indexer query scores every pooled key; each pooled key's importance becomes
     the running max of its old value and the new score; the new token's own
     importance is its self-score;
  2. the candidates are the pooled tokens outside the recent window p-R+1..p (the B
     older tokens plus the one leaving the window); the candidate with the lowest
     importance is evicted, ties evicting the higher position (the lower one is kept);
  3. the evicted K/V row is folded into M, b by one decayed rank-1 update per KV head;
  4. the new token takes the freed slot;
  5. the new query attends over the pool and adds the gated memory read-out.
"""
import numpy as np

from . import indexmem as im


class StreamState:
    def __init__(self, slot_pos, I, k_hat, Kc, Vc, M, b, next_pos, R):
        self.slot_pos = np.array(slot_pos, np.int64)
        self.I = np.array(I, np.float64)
        self.k_hat = np.array(k_hat, np.float64)
        self.Kc = np.array(Kc, np.float64)
        self.Vc = np.array(Vc, np.float64)
        self.M = np.array(M, np.float64)
        self.b = np.array(b, np.float64)
        self.next_pos = int(next_pos)
        self.R = int(R)


def from_prefill(pre: dict, L: int, R: int) -> StreamState:
    """Pool after pre-eviction: kept positions in ascending order occupy slots 0.."""
    idx = pre["idx"]
    return StreamState(idx, pre["I"][idx], pre["k_hat"][idx], pre["Kc"], pre["Vc"],
                       pre["M"], pre["b"], L, R)


def new_query_scores(q_hat, gate, k_hat):
    """Score of one indexer query (q_hat [H_I, d_I], gate [H_I]) against keys [n, d_I]:
    sum_h gate_h * relu(q_hat_h . k / sqrt(d_I))."""
    d_I = k_hat.shape[1]
    lg = np.maximum(np.asarray(k_hat, np.float64) @ np.asarray(q_hat, np.float64).T / np.sqrt(d_I), 0.0)
    return lg @ np.asarray(gate, np.float64)


def eviction_choice(I, pos, cand):
    """Index (into the pool) of the candidate with the lowest importance; among equal
    importances the higher position is evicted."""
    best = None
    for j in cand:
        key = (im.select_key(I[j]), -int(pos[j]))
        if best is None or key < best[0]:
            best = (key, j)
    return best[1]


def step(st: StreamState, x_new, q_new, k_new, v_new, W_kI, gamma_k, W_qI, gamma_q, W_g,
         w_g, lam, eps=1e-6, eps_mem=1e-6):
    """One streaming decode step (float64 inputs of one sequence).  x_new [D],
    q_new [H_q, d], k_new/v_new [H_kv, d].  Mutates st; returns (o [H_q, d], lse [H_q],
    evicted position, evicted slot)."""
    p = st.next_pos
    k_hat_new = im.indexer_keys(np.asarray(x_new)[None], W_kI, gamma_k, eps)[0]
    q_hat, gate = im.indexer_queries(np.asarray(q_new)[None], np.asarray(x_new)[None],
                                     W_qI, gamma_q, W_g, eps)
    st.I = np.maximum(st.I, new_query_scores(q_hat[0], gate[0], st.k_hat))
    I_new = new_query_scores(q_hat[0], gate[0], k_hat_new[None])[0]
    cand = [j for j in range(len(st.slot_pos)) if st.slot_pos[j] <= p - st.R]
    e = eviction_choice(st.I, st.slot_pos, cand)
    ev_pos = int(st.slot_pos[e])
    H_kv = st.Kc.shape[0]
    for g in range(H_kv):
        st.M[g], st.b[g] = im.memory_update_sequential(st.Kc[g, e][None], st.Vc[g, e][None],
                                                       lam, st.M[g], st.b[g])
    st.slot_pos[e] = p
    st.I[e] = I_new
    st.k_hat[e] = k_hat_new
    st.Kc[:, e] = k_new
    st.Vc[:, e] = v_new
    st.next_pos = p + 1
    d = st.Kc.shape[2]
    o, lse = im.decode_attention(q_new, st.Kc, st.Vc, st.Kc.shape[1], 1.0 / np.sqrt(d))
    m, g = im.memory_readout(q_new, st.M, st.b, w_g, eps_mem)
    return im.residual_output(o, m, g), lse, ev_pos, e
