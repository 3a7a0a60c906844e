"""MomentKV eviction during decode, fp64 reference -- TEST INFRASTRUCTURE ONLY.

The moment statistics are updated at every eviction [MKV part 1]. Here the cache is held
at a fixed pool of P slots per (sequence, KV head), and every decode step evicts one
token per KV head, chosen by the moment-informed score [MKV part 3]. The new query then
attends over the pool with the normalization-corrected mix [MKV part 4].

Reading (the pages give no per-step order). For the new token at position p, per KV head:
  1. alpha_j is the new query's softmax weight of pooled token j, averaged over the G
     query heads of the group. The softmax runs over the pool and the new token (what
     the query attends to). This is the prefill reading with a window of one query.
  2. score_j = alpha_j ||r_j||, with the moments accumulated so far.
  3. The candidates are the pooled tokens at positions <= p - R (R = 0: the whole pool).
     The lowest score is evicted; among equal scores the higher position goes, since the
     prefill keeps the lower one.
  4. The evicted K/V row is folded into (n_e, s_k, s_v, S).
  5. The new token takes the freed slot.
  6. The new query attends over the pool and mixes with the moment estimate.
"""
import math

import numpy as np

from . import indexmem as im
from . import momentkv as mk
from .streaming import eviction_choice


class MomentStreamState:
    """Per-sequence state: slot_pos [H_kv, P], Kc, Vc [H_kv, P, d], one moment dict per
    KV head, the next token's position and the recent window R."""

    def __init__(self, slot_pos, Kc, Vc, moms, next_pos, R):
        self.slot_pos = np.array(slot_pos, np.int64)
        self.Kc = np.array(Kc, np.float64)
        self.Vc = np.array(Vc, np.float64)
        self.moms = [dict(n=int(m["n"]), sk=np.array(m["sk"], np.float64), sv=np.array(m["sv"], np.float64),
                          S=np.array(m["S"], np.float64)) for m in moms]
        self.next_pos = int(next_pos)
        self.R = int(R)


def from_prefill(pre: dict, K, V, L: int, R: int) -> MomentStreamState:
    """Pool after the moment-informed prefill (mk.prefill): each KV head's kept positions,
    in ascending order, occupy slots 0..B-1.  K, V [L, H_kv, d]."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    heads = pre["heads"]
    pos = np.stack([h["kept"] for h in heads])
    Kc = np.stack([K[h["kept"], g] for g, h in enumerate(heads)])
    Vc = np.stack([V[h["kept"], g] for g, h in enumerate(heads)])
    return MomentStreamState(pos, Kc, Vc, [h["mom"] for h in heads], L, R)


def step_alpha(q_grp, Kpool, k_new, scale):
    """Reading 1: alpha over the pool for one KV group.  q_grp [G, d], Kpool [P, d],
    k_new [d] -> [P].  The new token's own weight is part of every softmax row but is not
    returned."""
    q_grp = np.asarray(q_grp, np.float64)
    keys = np.vstack([np.asarray(Kpool, np.float64), np.asarray(k_new, np.float64)[None]])
    al = np.zeros(keys.shape[0])
    for q in q_grp:
        logit = scale * (keys @ q)
        w = np.exp(logit - logit.max())
        al += w / w.sum()
    return al[:-1] / q_grp.shape[0]


def step(st: MomentStreamState, q, k_new, v_new):
    """One decode step of one sequence.  q [H_q, d], k_new/v_new [H_kv, d] (float64).
    Mutates st.  Returns (o [H_q, d], lse_R [H_q], evicted slots [H_kv], evicted
    positions [H_kv], scores [H_kv, P] of the pool before the hand-over)."""
    q = np.asarray(q, np.float64)
    H_q, d = q.shape
    H_kv, P, _ = st.Kc.shape
    G = H_q // H_kv
    scale = 1.0 / math.sqrt(d)
    p = st.next_pos
    slots, ev_pos, scores = [], [], []
    for g in range(H_kv):
        al = step_alpha(q[g * G:(g + 1) * G], st.Kc[g], k_new[g], scale)
        sc = mk.score(al, st.Kc[g], st.Vc[g], st.moms[g], d)
        cand = [j for j in range(P) if st.slot_pos[g, j] <= p - st.R]
        e = eviction_choice(sc, st.slot_pos[g], cand)
        st.moms[g] = mk.add(st.moms[g], st.Kc[g, e], st.Vc[g, e])
        ev_pos.append(int(st.slot_pos[g, e]))
        st.slot_pos[g, e] = p
        st.Kc[g, e] = k_new[g]
        st.Vc[g, e] = v_new[g]
        slots.append(e)
        scores.append(sc)
    st.next_pos = p + 1
    out = np.zeros((H_q, d))
    lse = np.zeros(H_q)
    for h in range(H_q):
        g = h // G
        f_R, lse[h] = im.attention_state(q[h], st.Kc[g], st.Vc[g], scale)
        out[h], _ = mk.mix(q[h], f_R, lse[h], st.moms[g], d)
    return out, lse, np.array(slots), np.array(ev_pos), np.array(scores)
