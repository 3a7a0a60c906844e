"""Plant plausible mistakes in the oracle (CPU only) and check that a pin catches each.

Every mutation below is a slip that could be made when writing the method down from
the pages: a dropped term, a transposed operand, a reversed order, a wrong index.
"""
import numpy as np
import pytest

from oracle import indexmem as im
from oracle import asm
from oracle import chunked as ck
from oracle import moment_stream as ms
from oracle import momentkv as mk
from oracle import streaming as sm
from tests import test_oracle_golden as gold
from tests import test_oracle_pins as pins

_orig = {name: getattr(im, name) for name in dir(im) if callable(getattr(im, name))}
_orig_mk = {name: getattr(mk, name) for name in dir(mk) if callable(getattr(mk, name))}
_orig_ms = {name: getattr(ms, name) for name in dir(ms) if callable(getattr(ms, name))}
_orig_asm = {name: getattr(asm, name) for name in dir(asm) if callable(getattr(asm, name))}
_orig_ck = {name: getattr(ck, name) for name in dir(ck) if callable(getattr(ck, name))}
_orig_sm = {name: getattr(sm, name) for name in dir(sm) if callable(getattr(sm, name))}


def _phi_no_plus_one(x):
    x = np.asarray(x, np.float64)
    return np.where(x > 0, x, np.exp(np.minimum(x, 0.0)))


def _memory_transposed(K_ev, V_ev, lam, M0=None, b0=None):
    M, b = _orig["memory_build"](K_ev, V_ev, lam, M0, b0)
    return M.T, b


def _memory_reversed_decay(K_ev, V_ev, lam, M0=None, b0=None):
    return _orig["memory_build"](np.asarray(K_ev)[::-1], np.asarray(V_ev)[::-1], lam, M0, b0)


def _score_mask_flipped(q_hat, gate, k_hat, q_pos, act="relu"):
    A = _orig["score_matrix"](q_hat, gate, k_hat, np.full(len(q_pos), k_hat.shape[0]), act)
    L = k_hat.shape[0]
    mask = np.arange(L)[None, :] < np.asarray(q_pos)[:, None] - 1
    return np.where(mask, -np.inf, A)


def _score_relu_after_sum(q_hat, gate, k_hat, q_pos, act="relu"):
    A = _orig["score_matrix"](q_hat, gate, k_hat, q_pos, "none")
    return np.where(np.isneginf(A), A, np.maximum(A, 0.0)) if act == "relu" else A


def _score_no_scale(q_hat, gate, k_hat, q_pos, act="relu"):
    return _orig["score_matrix"](q_hat, gate, k_hat, q_pos, act) * np.sqrt(k_hat.shape[1])


def _topk_tie_high(I, B, R=0, recent_inclusive=True):
    L = len(I)
    rev = np.asarray(I)[::-1]
    # select on the reversed array (ties then prefer the original higher position)
    idx, _ = _orig["topk_select"](rev, B, 0, recent_inclusive) if R == 0 else (None, None)
    if idx is None:
        return _orig["topk_select"](I, B, R, recent_inclusive)
    kept = sorted(L - 1 - idx)
    sm = np.zeros(L, np.int64)
    s = e = 0
    for t in range(L):
        if t in kept:
            sm[t] = s
            s += 1
        else:
            e += 1
            sm[t] = -e
    return np.array(kept), sm


def _merge_unweighted(states):
    lses = np.array([l for _, l in states])
    a = sum(ai for ai, _ in states) / len(states)
    return a, np.log(np.sum(np.exp(lses)))


def _gqa_modulo(q, Kc, Vc, n, scale):
    q = np.asarray(q, np.float64)
    H_kv = Kc.shape[0]
    o = np.zeros_like(q)
    lse = np.zeros(q.shape[0])
    for h in range(q.shape[0]):
        o[h], lse[h] = _orig["attention_state"](q[h], Kc[h % H_kv, :n], Vc[h % H_kv, :n], scale)
    return o, lse


def _readout_transposed(q, M, b, w_g, eps=1e-6):
    return _orig["memory_readout"](q, np.swapaxes(M, 1, 2), b, w_g, eps)


def _stats_unscaled(mom):
    kbar, vbar, St = _orig_mk["stats"](mom)
    return kbar, vbar, mom["S"] - np.outer(mom["sv"], mom["sk"])


def _estimate_no_sqrt(q, mom, d):
    _, vbar, St = mk.stats(mom)
    return vbar + St @ np.asarray(q, np.float64) / mom["n"]


def _logz_no_count(q, mom, d):
    return _orig_mk["log_Z_hat"](q, mom, d) - np.log(mom["n"])


def _residual_plus(k, v, mom, d):
    if mom["n"] == 0:
        return np.asarray(v, np.float64).copy()
    _, vbar, St = mk.stats(mom)
    return np.asarray(v) - vbar + (np.asarray(k) @ St.T) / (mom["n"] * np.sqrt(d))


def _stream_alpha_without_new(q_grp, Kpool, k_new, scale):
    q_grp = np.asarray(q_grp, np.float64)
    al = np.zeros(len(Kpool))
    for q in q_grp:
        lg = scale * (np.asarray(Kpool) @ q)
        w = np.exp(lg - lg.max())
        al += w / w.sum()
    return al / len(q_grp)


def _evict_highest(scores, pos, cand):
    return _orig_ms["eviction_choice"]([-x for x in scores], pos, cand)


def _evict_lower_on_ties(scores, pos, cand):
    return min(cand, key=lambda j: (im.select_key(scores[j]), int(pos[j])))


def _mq_transposed(q, W_m):
    return _orig["memory_query"](q, np.asarray(W_m).T)


def _readout_gate_on_projection(q, M, b, w_g, eps=1e-6, q_mem=None):
    return _orig["memory_readout"](q if q_mem is None else q_mem, M, b, w_g, eps, q_mem)


def _readout_projection_after_phi(q, M, b, w_g, eps=1e-6, q_mem=None):
    # W phi(q) instead of phi(W q); W is recovered from (q, q_mem) by least squares
    if q_mem is None:
        return _orig["memory_readout"](q, M, b, w_g, eps)
    q = np.asarray(q, np.float64)
    W = np.linalg.lstsq(q, np.asarray(q_mem, np.float64), rcond=None)[0].T
    H_q, G = q.shape[0], q.shape[0] // M.shape[0]
    m = np.zeros_like(q)
    g = np.zeros(H_q)
    for h in range(H_q):
        f = W @ im.phi(q[h])
        m[h] = (M[h // G] @ f) / (b[h // G] @ f + eps)
        g[h] = im.sigmoid(np.asarray(w_g)[h] @ q[h])
    return m, g


def _aggregate_plain_mean(a, lse, idx, K):
    a = np.asarray(a, np.float64)
    a_bar, lse_bar = _orig_asm["aggregate"](a, lse, idx, K)
    for k in range(K):
        if (idx == k).any():
            a_bar[k] = a[idx == k].mean(0)
    return a_bar, lse_bar


def _aggregate_summed_partition(a, lse, idx, K):
    a_bar, lse_bar = _orig_asm["aggregate"](a, lse, idx, K)
    for k in range(K):
        n = int((idx == k).sum())
        if n:
            lse_bar[k] += np.log(n)
    return a_bar, lse_bar


def _lookup_dot(q, C):
    return int(np.argmax(np.asarray(C) @ np.asarray(q)))


def _assign_farthest(X, C):
    idx, d2 = _orig_asm["kmeans_assign"](X, C)
    return np.argmax(d2, axis=1), d2


def _chunked_window_at_start(X, Q, K, V, W_kI, gamma_k, W_qI, gamma_q, W_g, B, R, lam, C, W,
                             recent_inclusive=True, act="relu", eps=1e-6):
    # the window read at each chunk's first W positions instead of its last W
    Qs = np.array(Q, np.float64)
    Xs = np.array(X, np.float64)
    L = Xs.shape[0]
    for s0 in range(0, L, C):
        e = min(L, s0 + C)
        Qs[e - W:e], Xs[e - W:e] = np.array(Q[s0:s0 + W]), np.array(X[s0:s0 + W])
    return _orig_ck["prefill_chunked"](Xs, Qs, K, V, W_kI, gamma_k, W_qI, gamma_q, W_g, B, R, lam, C, W,
                                       recent_inclusive, act, eps)


def _select_lowest(scores, pos, keep):
    # each MomentKV round keeps the lowest scores instead of the highest
    return _orig_mk["select_round"](-np.asarray(scores, np.float64), pos, keep)


def _score_empty_moments(alpha_j, k, v, mom, d):
    # every round scored as if nothing had been evicted yet
    return _orig_mk["score"](alpha_j, k, v, mk.empty(d), d)


def _mk_decode_no_append(q_steps, k_steps, v_steps, K, V, heads, T=None):
    # the decode attends over the kept rows only: the new K/V never joins them
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    T = q_steps.shape[0] if T is None else T
    H_q, d = q_steps.shape[1], q_steps.shape[2]
    G = H_q // K.shape[1]
    out, lses, ws = np.zeros((T, H_q, d)), np.zeros((T, H_q)), np.zeros((T, H_q))
    for t in range(T):
        for h in range(H_q):
            g = h // G
            q = np.asarray(q_steps[t, h], np.float64)
            f_R, lse_R = im.attention_state(q, K[heads[g]["kept"], g], V[heads[g]["kept"], g], d ** -0.5)
            out[t, h], ws[t, h] = mk.mix(q, f_R, lse_R, heads[g]["mom"], d)
            lses[t, h] = lse_R
    return out, lses, ws


def _stream_readout_before_fold(st, x_new, q_new, k_new, v_new, W_kI, gamma_k, W_qI, gamma_q, W_g,
                                w_g, lam, eps=1e-6, eps_mem=1e-6):
    # the step reads the memory out with M, b from before the evicted row's fold
    M0, b0 = st.M.copy(), st.b.copy()
    o, lse, ev, e = _orig_sm["step"](st, x_new, q_new, k_new, v_new, W_kI, gamma_k, W_qI, gamma_q,
                                     W_g, w_g, lam, eps, eps_mem)
    m1, g = im.memory_readout(q_new, st.M, st.b, w_g, eps_mem)
    m0, _ = im.memory_readout(q_new, M0, b0, w_g, eps_mem)
    return o - g[:, None] * m1 + g[:, None] * m0, lse, ev, e


def _residual_without_gate(o_attn, m, g):
    return o_attn + m


MUTATIONS_COMPOSITION = [
    ("MomentKV round keeps the lowest scores", mk, "select_round", _select_lowest,
     [pins.test_moment_rounds_selection_and_residuals_brute_force]),
    ("MomentKV later rounds scored with empty moments", mk, "score", _score_empty_moments,
     [pins.test_moment_rounds_selection_and_residuals_brute_force]),
    ("MomentKV decode does not append the new K/V", mk, "decode", _mk_decode_no_append,
     [lambda: pins.test_momentkv_decode_appends_then_mixes_brute_force(5),
      lambda: pins.test_momentkv_decode_appends_then_mixes_brute_force(60)]),
    ("stream step reads the memory before the fold", sm, "step", _stream_readout_before_fold,
     [pins.test_streaming_step_output_brute_force]),
    ("decode drops the memory gate", im, "residual_output", _residual_without_gate,
     [pins.test_indexmem_decode_with_memory_brute_force]),
]


MUTATIONS_STREAM = [
    ("stream alpha drops the new token", ms, "step_alpha", _stream_alpha_without_new,
     [pins.test_stream_alpha_is_textbook_softmax_and_window_of_one]),
    ("stream evicts the highest score", ms, "eviction_choice", _evict_highest,
     [pins.test_stream_step_hand_example, pins.test_stream_steps_brute_force_choice_and_moments]),
    ("stream ties evict the lower position", ms, "eviction_choice", _evict_lower_on_ties,
     [pins.test_stream_step_hand_example]),
    ("read-out projection transposed", im, "memory_query", _mq_transposed,
     [pins.test_memory_query_projection_special_cases]),
    ("gate reads the projected query", im, "memory_readout", _readout_gate_on_projection,
     [pins.test_memory_query_projection_special_cases]),
    ("projection applied after phi", im, "memory_readout", _readout_projection_after_phi,
     [pins.test_memory_query_projection_special_cases]),
    ("ASM state: plain mean of outputs", asm, "aggregate", _aggregate_plain_mean,
     [pins.test_asm_aggregate_is_partition_weighted_mean]),
    ("ASM state: summed partition", asm, "aggregate", _aggregate_summed_partition,
     [pins.test_asm_aggregate_is_partition_weighted_mean]),
    ("ASM lookup by dot product", asm, "lookup", _lookup_dot, [pins.test_asm_lookup_is_cosine_argmax]),
    ("K-means assigns the farthest", asm, "kmeans_assign", _assign_farthest, [pins.test_kmeans_lloyd_steps]),
    ("chunk window at the chunk's start", ck, "prefill_chunked", _chunked_window_at_start,
     [pins.test_chunked_single_chunk_is_one_shot_prefill, pins.test_chunked_running_max_budget_and_fold_composition]),
]


MUTATIONS = [
    ("phi drops +1", im, "phi", _phi_no_plus_one, [pins.test_phi_is_elu_plus_one, gold.test_memory_tiny]),
    ("M transposed", im, "memory_build", _memory_transposed, [pins.test_memory_special_cases, gold.test_memory_tiny]),
    ("decay order reversed", im, "memory_build", _memory_reversed_decay,
     [lambda: pins.test_memory_closed_form_equals_recurrence(0.5), gold.test_memory_tiny]),
    ("causal mask flipped", im, "score_matrix", _score_mask_flipped,
     [lambda: pins.test_importance_brute_force_and_streaming("relu"), gold.test_indexer_tiny]),
    ("ReLU after head sum", im, "score_matrix", _score_relu_after_sum, [pins.test_relu_is_per_head_before_the_gated_sum]),
    ("logit scale dropped", im, "score_matrix", _score_no_scale, [pins.test_indexer_logit_is_scaled_cosine, gold.test_indexer_tiny]),
    ("ties keep higher position", im, "topk_select", _topk_tie_high, [gold.test_indexer_tiny]),
    ("merge ignores Z", im, "merge_states", _merge_unweighted, [lambda: pins.test_split_merge_equals_unsplit(0)]),
    ("GQA head map h % H_kv", im, "decode_attention", _gqa_modulo, [pins.test_decode_attention_gqa_mapping]),
    ("read-out uses M^T", im, "memory_readout", _readout_transposed, [pins.test_readout_special_cases, gold.test_memory_tiny]),
    ("S~ missing 1/n_e", mk, "stats", _stats_unscaled, [pins.test_moment_stats_brute_force_and_additivity, gold.test_moments_tiny]),
    ("estimate missing sqrt d", mk, "evicted_estimate", _estimate_no_sqrt, [pins.test_moment_estimate_is_linearised_softmax]),
    ("Z^ missing n_e", mk, "log_Z_hat", _logz_no_count, [gold.test_moments_tiny]),
    ("residual sign flipped", mk, "residual", _residual_plus,
     [gold.test_moments_tiny, pins.test_residual_is_value_minus_estimate_at_its_key]),
]


ALL_MUTATIONS = MUTATIONS + MUTATIONS_STREAM + MUTATIONS_COMPOSITION


@pytest.mark.parametrize("name,mod,attr,fn,tests", ALL_MUTATIONS, ids=[m[0] for m in ALL_MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, mod, attr, fn, tests):
    monkeypatch.setattr(mod, attr, fn)
    for t in tests:
        with pytest.raises(Exception):
            t()
