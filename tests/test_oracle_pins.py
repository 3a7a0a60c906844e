"""The oracle pinned to things other than itself: closed forms, textbook special cases,
invariants and brute force on tiny inputs.  Each test names the mistake it catches."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.special import softmax as sp_softmax, logsumexp as sp_lse

from oracle import asm
from oracle import chunked as ck
from oracle import indexmem as im
from oracle import moment_stream as ms
from oracle import momentkv as mk
from oracle import streaming as sm

R = np.random.default_rng(12345)


def rnd(*shape, scale=1.0, seed=None):
    r = R if seed is None else np.random.default_rng(seed)
    return r.standard_normal(shape) * scale


# ============================================================================ phi, norm, gate

def test_phi_is_elu_plus_one():
    # catches: a wrong branch, a missing +1, exp on the positive side
    xs = np.array([-30.0, -2.0, -1e-9, 0.0, 1e-9, 0.5, 7.0])
    want = [math.exp(-30.0), math.exp(-2.0), math.exp(-1e-9), 1.0, 1.0 + 1e-9, 1.5, 8.0]
    np.testing.assert_allclose(im.phi(xs), want, rtol=1e-15)
    assert np.all(im.phi(rnd(1000) * 10) > 0)


def test_rmsnorm_unit_rms_and_gamma():
    x = rnd(5, 32)
    y = im.rmsnorm(x, np.ones(32), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), 1.0, rtol=1e-13)
    gam = rnd(32)
    np.testing.assert_allclose(im.rmsnorm(x, gam, 0.0), y * gam, rtol=1e-13)
    np.testing.assert_allclose(im.rmsnorm(3.0 * x, np.ones(32), 0.0), y, rtol=1e-13)


def test_indexer_logit_is_scaled_cosine():
    # With gamma = 1 and eps = 0, q_hat.k_hat/sqrt(d_I) = sqrt(d_I) cos(qI, kI): the textbook
    # cosine, computed here by explicit loops from the raw projections.
    D, d, dI, H_I, W, L = 12, 8, 4, 2, 3, 5
    X, Q = rnd(L, D), rnd(W, 1, d)
    WkI, WqI, Wg = rnd(dI, D), rnd(H_I, dI, d), np.zeros((H_I, D))
    kh = im.indexer_keys(X, WkI, np.ones(dI), 0.0)
    qh, gate = im.indexer_queries(Q, X[L - W:], WqI, np.ones(dI), Wg, 0.0)
    A = im.score_matrix(qh, gate, kh, np.full(W, L - 1), act="none")
    for s in range(W):
        for t in range(L):
            tot = 0.0
            for h in range(H_I):
                kI = [sum(WkI[i, j] * X[t, j] for j in range(D)) for i in range(dI)]
                qI = [sum(WqI[h, i, j] * Q[s, 0, j] for j in range(d)) for i in range(dI)]
                cos = sum(a * b for a, b in zip(qI, kI)) / (math.sqrt(sum(a * a for a in qI)) *
                                                           math.sqrt(sum(b * b for b in kI)))
                tot += 0.5 * math.sqrt(dI) * cos      # W_g = 0 -> gate = 1/2
            assert math.isclose(A[s, t], tot, rel_tol=1e-12)


def test_gate_values():
    # catches: gate on the wrong operand, missing sigmoid
    x = np.array([[1.0, 0.0]])
    Wg = np.array([[math.log(3.0), 5.0]])
    _, g = im.indexer_queries(rnd(1, 1, 4), x, rnd(1, 2, 4), np.ones(2), Wg)
    assert math.isclose(g[0, 0], 0.75, rel_tol=1e-15)
    _, g0 = im.indexer_queries(rnd(1, 1, 4), rnd(1, 7), rnd(3, 2, 4), np.ones(2), np.zeros((3, 7)))
    assert np.all(g0 == 0.5)


def test_indexer_head_map_reads_the_right_query_head():
    # H_I = 4 indexer heads over H_q = 2 model heads: heads 0,1 read model head 0, 2,3 head 1
    assert im.indexer_head_map(4, 2) == [0, 0, 1, 1]
    assert im.indexer_head_map(4, 1) == [0, 0, 0, 0]
    assert im.indexer_head_map(32, 32) == list(range(32))
    Q = rnd(2, 2, 6)
    WqI = rnd(4, 3, 6)
    q1, _ = im.indexer_queries(Q, rnd(2, 5), WqI, np.ones(3), rnd(4, 5))
    Q2 = Q.copy()
    Q2[:, 1] += 1.0           # change model head 1 only
    q2, _ = im.indexer_queries(Q2, rnd(2, 5), WqI, np.ones(3), rnd(4, 5))
    np.testing.assert_array_equal(q1[:, :2], q2[:, :2])
    assert np.all(np.abs(q1[:, 2:] - q2[:, 2:]) > 0)


# ============================================================================ A3 score + pool

def _brute_importance(qh, gate, kh, qpos, act):
    W, H, dI = qh.shape
    L = kh.shape[0]
    I = [-math.inf] * L
    for t in range(L):
        for s in range(W):
            if t > qpos[s]:
                continue
            a = 0.0
            for h in range(H):
                lg = sum(qh[s, h, i] * kh[t, i] for i in range(dI)) / math.sqrt(dI)
                a += gate[s, h] * (max(lg, 0.0) if act == "relu" else lg)
            I[t] = max(I[t], a)
    return np.array(I)


@pytest.mark.parametrize("act", ["relu", "none"])
def test_importance_brute_force_and_streaming(act):
    # catches: a wrong causal mask direction, sum/max order swapped, ReLU after the head sum
    W, H, dI, L = 4, 3, 5, 9
    qh, gate, kh = rnd(W, H, dI), 1 / (1 + np.exp(-rnd(W, H))), rnd(L, dI)
    qpos = np.arange(L - W, L)
    I = im.importance(im.score_matrix(qh, gate, kh, qpos, act))
    np.testing.assert_allclose(I, _brute_importance(qh, gate, kh, qpos, act), rtol=1e-12)
    np.testing.assert_allclose(im.importance_streaming(qh, gate, kh, qpos, act), I, rtol=0, atol=0)


def test_relu_is_per_head_before_the_gated_sum():
    qh = np.array([[[1.0, 0.0], [-1.0, 0.0]]])     # head logits +1/sqrt2 and -1/sqrt2
    A = im.score_matrix(qh, np.ones((1, 2)), np.array([[1.0, 0.0]]), np.array([0]))
    assert math.isclose(A[0, 0], 1 / math.sqrt(2), rel_tol=1e-15)


def test_linear_form_collapses_to_one_vector():
    # act = none: A[s,t] = (sum_h g q_hat_h) . k_hat / sqrt(d_I)
    W, H, dI, L = 3, 4, 6, 7
    qh, gate, kh = rnd(W, H, dI), rnd(W, H) ** 2, rnd(L, dI)
    qpos = np.full(W, L - 1)
    A = im.score_matrix(qh, gate, kh, qpos, act="none")
    qs = np.einsum("sh,shi->si", gate, qh)
    np.testing.assert_allclose(A, qs @ kh.T / math.sqrt(dI), rtol=1e-12)


def test_window_of_one_is_last_row_and_gate_scales():
    W, H, dI, L = 1, 3, 4, 6
    qh, kh = rnd(W, H, dI), rnd(L, dI)
    I1 = im.importance(im.score_matrix(qh, np.ones((1, H)), kh, np.array([L - 1])))
    I2 = im.importance(im.score_matrix(qh, np.full((1, H), 0.5), kh, np.array([L - 1])))
    np.testing.assert_allclose(I2, I1 / 2, rtol=1e-15)
    manual = [sum(max(qh[0, h] @ kh[t] / 2.0, 0) for h in range(H)) for t in range(L)]
    np.testing.assert_allclose(I1, manual, rtol=1e-13)


# ============================================================================ A4 top-k

def _check_selection(I, B, R, inclusive, idx, smap):
    L = len(I)
    n_top = B - R if inclusive else B
    Rr = min(R, L)
    cand = range(L - Rr)
    kept = set(idx.tolist())
    keyf = lambda t: (-(-math.inf if math.isnan(I[t]) else float(I[t]) + 0.0), t)
    if n_top >= L - Rr:
        assert kept == set(range(L))
    else:
        assert len(kept) == n_top + Rr
        assert all(t in kept for t in range(L - Rr, L))
        ck = [t for t in cand if t in kept]
        ce = [t for t in cand if t not in kept]
        for a in ck:
            for e in ce:
                assert keyf(a) < keyf(e)
    assert list(idx) == sorted(idx)
    slots = [smap[t] for t in range(L) if t in kept]
    assert slots == list(range(len(kept)))
    ranks = [-smap[t] for t in range(L) if t not in kept]
    assert ranks == list(range(1, L - len(kept) + 1))


@settings(max_examples=60, deadline=None)
@given(L=st.integers(1, 40), B=st.integers(0, 45), R=st.integers(0, 8), inclusive=st.booleans(),
       levels=st.sampled_from([0, 2, 5]), seed=st.integers(0, 10 ** 6))
def test_topk_against_pairwise_definition(L, B, R, inclusive, levels, seed):
    if inclusive and B < R:
        B = R
    x = np.random.default_rng(seed).standard_normal(L)
    if levels:
        x = np.floor(x * levels) / levels
    idx, smap = im.topk_select(x, B, R, inclusive)
    _check_selection(x, B, R, inclusive, idx, smap)


def test_topk_special_values():
    I = np.array([np.nan, 1.0, -0.0, 0.0, -np.inf, np.nan, 0.0])
    idx, _ = im.topk_select(I, 3, 0)
    # order: 1.0 (t=1), then the zeros t=2 (-0), t=3, t=6; -0 ties +0 -> lowest positions
    assert idx.tolist() == [1, 2, 3]
    # NaN orders as -inf and ties the real -inf (t=4): of t=0, 4, 5 the lowest two are kept
    idx, _ = im.topk_select(I, 6, 0)
    assert idx.tolist() == [0, 1, 2, 3, 4, 6]


def test_topk_budget_edges():
    I = rnd(20)
    idx, smap = im.topk_select(I, 20, 0)
    assert idx.tolist() == list(range(20)) and smap.tolist() == list(range(20))
    idx, smap = im.topk_select(I, 4, 4)           # budget = recent window
    assert idx.tolist() == [16, 17, 18, 19]
    idx, _ = im.topk_select(I, 5, 4, recent_inclusive=False)
    assert len(idx) == 9 and idx[-4:].tolist() == [16, 17, 18, 19]


def test_topk_permutation_equivariant():
    I = rnd(30)
    perm = R.permutation(30)
    idx, _ = im.topk_select(I, 7, 0)
    idx2, _ = im.topk_select(I[perm], 7, 0)
    assert sorted(perm[idx2].tolist()) == idx.tolist()


# ============================================================================ A5 compaction

def test_compact_gathers_bit_exactly():
    L, H, d = 11, 3, 4
    K = R.integers(0, 65535, (L, H, d)).astype(np.uint16)
    V = R.integers(0, 65535, (L, H, d)).astype(np.uint16)
    idx, smap = im.topk_select(rnd(L), 5, 2)
    Kc, Vc = im.compact(K, V, smap, 8)
    for s, t in enumerate(idx):
        for g in range(H):
            assert Kc[g, s].tobytes() == K[t, g].tobytes()
            assert Vc[g, s].tobytes() == V[t, g].tobytes()
    assert not Kc[:, 5:].any()
    idx, smap = im.topk_select(rnd(L), L, 0)
    Kc, _ = im.compact(K, V, smap, L)
    assert np.array_equal(Kc, K.transpose(1, 0, 2))


def test_evicted_order_is_ascending_position():
    _, smap = im.topk_select(np.array([5.0, 1.0, 4.0, 0.5, 3.0, 0.1]), 2, 0)
    assert im.evicted_in_order(smap).tolist() == [1, 3, 4, 5]


# ============================================================================ A6 memory

@pytest.mark.parametrize("lam", [0.0, 0.5, 0.99, 1.0])
def test_memory_closed_form_equals_recurrence(lam):
    n, d = 37, 6
    K, V = rnd(n, d, scale=2), rnd(n, d)
    M0, b0 = rnd(d, d), rnd(d)
    M, b = im.memory_build(K, V, lam, M0, b0)
    Ms, bs = im.memory_update_sequential(K, V, lam, M0, b0)
    np.testing.assert_allclose(M, Ms, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b, bs, rtol=1e-12, atol=1e-12)


def test_memory_special_cases():
    d = 5
    k, v = rnd(1, d), rnd(1, d)
    M, b = im.memory_build(k, v, 0.9)
    f = [math.exp(x) if x <= 0 else x + 1 for x in k[0]]
    for i in range(d):
        for j in range(d):
            assert M[i, j] == pytest.approx(v[0, i] * f[j], rel=1e-15)   # rows index v
    K, V = rnd(9, d), rnd(9, d)
    M1, b1 = im.memory_build(K, V, 1.0)
    np.testing.assert_allclose(M1, sum(np.outer(V[i], im.phi(K[i])) for i in range(9)), rtol=1e-13)
    M0_, b0_ = im.memory_build(K, V, 0.0)
    np.testing.assert_allclose(M0_, np.outer(V[-1], im.phi(K[-1])), rtol=1e-15)
    np.testing.assert_allclose(b0_, im.phi(K[-1]), rtol=1e-15)


def test_memory_split_composition():
    # build(E1 u E2) = lam^|E2| build(E1) + build(E2): the rule any split-K build obeys
    K, V = rnd(50, 4), rnd(50, 4)
    lam = 0.97
    M, b = im.memory_build(K, V, lam)
    Ma, ba = im.memory_build(K[:23], V[:23], lam)
    Mb, bb = im.memory_build(K[23:], V[23:], lam)
    np.testing.assert_allclose(M, lam ** 27 * Ma + Mb, rtol=1e-12)
    np.testing.assert_allclose(b, lam ** 27 * ba + bb, rtol=1e-12)


# ============================================================================ A8 attention

def test_attention_state_is_textbook_softmax():
    q, K, V = rnd(8), rnd(13, 8), rnd(13, 8)
    a, lse = im.attention_state(q, K, V, 0.3)
    np.testing.assert_allclose(a, sp_softmax(0.3 * K @ q) @ V, rtol=1e-12)
    assert math.isclose(lse, sp_lse(0.3 * K @ q), rel_tol=1e-13)
    a1, l1 = im.attention_state(q, K[:1], V[:1], 0.3)
    np.testing.assert_array_equal(a1, V[0])
    assert math.isclose(l1, 0.3 * K[0] @ q, rel_tol=1e-14)


@pytest.mark.parametrize("seed", range(5))
def test_split_merge_equals_unsplit(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(1, 60))
    q, K, V = r.standard_normal(16) * 3, r.standard_normal((n, 16)), r.standard_normal((n, 16))
    cuts = np.sort(r.integers(0, n + 1, int(r.integers(0, 6))))
    bounds = [0, *cuts.tolist(), n]
    states = [im.attention_state(q, K[a:b], V[a:b], 0.25) for a, b in zip(bounds[:-1], bounds[1:])]
    a, lse = im.merge_states(states)
    a0, l0 = im.attention_state(q, K, V, 0.25)
    np.testing.assert_allclose(a, a0, rtol=1e-12, atol=1e-14)
    assert math.isclose(lse, l0, rel_tol=1e-13)
    perm = r.permutation(n)
    ap, lp = im.attention_state(q, K[perm], V[perm], 0.25)
    np.testing.assert_allclose(ap, a0, rtol=1e-12, atol=1e-14)


def test_decode_attention_gqa_mapping():
    Kc, Vc = rnd(2, 5, 4), rnd(2, 5, 4)
    q = rnd(4, 4)
    o, _ = im.decode_attention(q, Kc, Vc, 5, 0.5)
    for h in range(4):
        np.testing.assert_allclose(o[h], sp_softmax(0.5 * Kc[h // 2] @ q[h]) @ Vc[h // 2], rtol=1e-12)


# ============================================================================ A9 readout

def test_readout_special_cases():
    q = rnd(4, 6)
    M, b = np.zeros((2, 6, 6)), np.zeros((2, 6))
    m, g = im.memory_readout(q, M, b, rnd(4, 6))
    assert np.all(m == 0)
    o = rnd(4, 6)
    np.testing.assert_array_equal(im.residual_output(o, m, g), o)
    # one evicted token: m = v (phi(k).phi(q)) / (phi(k).phi(q) + eps)
    k, v = rnd(6), rnd(6)
    M1, b1 = im.memory_build(k[None], v[None], 0.9)
    m1, _ = im.memory_readout(q[:1], M1[None], b1[None], np.zeros((1, 6)), eps=1e-6)
    dot = sum((math.exp(a) if a <= 0 else a + 1) * (math.exp(c) if c <= 0 else c + 1)
              for a, c in zip(k, q[0]))
    np.testing.assert_allclose(m1[0], v * dot / (dot + 1e-6), rtol=1e-13)
    # gate -> 0 removes the memory term
    _, g0 = im.memory_readout(q[:1], M1[None], b1[None], -1e4 * np.sign(q[:1]))
    assert g0[0] < 1e-300


# ============================================================================ end to end

def _full_attention(q, K, V, scale):
    s = [scale * sum(a * b for a, b in zip(q, k)) for k in K]
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    Z = sum(e)
    return np.array([sum(e[j] * V[j][i] for j in range(len(K))) / Z for i in range(len(q))])


def test_no_eviction_equals_full_attention():
    # B = L: nothing is evicted, M = 0, b = 0, and decode equals full attention
    L, D, Hq, Hkv, d, dI, HI, W, T = 24, 16, 4, 2, 8, 4, 4, 5, 3
    X, Q, K, V = rnd(L, D), rnd(W, Hq, d), rnd(L, Hkv, d), rnd(L, Hkv, d)
    pre = im.prefill(X, Q, K, V, rnd(dI, D), np.ones(dI), rnd(HI, dI, d), np.ones(dI),
                     rnd(HI, D), B=L, R=2, lam=0.9, cap=L + T)
    assert pre["n_evicted"] == 0 and not pre["M"].any() and not pre["b"].any()
    qs, ks, vs = rnd(T, Hq, d), rnd(T, Hkv, d), rnd(T, Hkv, d)
    o, _, _, _ = im.decode(qs, ks, vs, pre["Kc"], pre["Vc"], L, pre["M"], pre["b"], rnd(Hq, d))
    for t in range(T):
        for h in range(Hq):
            g = h // 2
            Kf = [*K[:, g].tolist(), *ks[:t + 1, g].tolist()]
            Vf = [*V[:, g].tolist(), *vs[:t + 1, g].tolist()]
            np.testing.assert_allclose(o[t, h], _full_attention(qs[t, h], Kf, Vf, d ** -0.5),
                                       rtol=1e-11, atol=1e-13)


def test_prefill_pipeline_consistency():
    L, D, Hq, Hkv, d, dI, HI, W = 40, 16, 4, 2, 8, 4, 4, 6
    X, Q, K, V = rnd(L, D), rnd(W, Hq, d), rnd(L, Hkv, d), rnd(L, Hkv, d)
    pre = im.prefill(X, Q, K, V, rnd(dI, D), np.ones(dI), rnd(HI, dI, d), np.ones(dI),
                     rnd(HI, D), B=10, R=3, lam=0.95)
    assert pre["n_kept"] == 10 and pre["n_evicted"] == 30
    ev = [t for t in range(L) if t not in set(pre["idx"].tolist())]
    for g in range(Hkv):
        Ms, bs = im.memory_update_sequential(K[ev, g], V[ev, g], 0.95, np.zeros((d, d)), np.zeros(d))
        np.testing.assert_allclose(pre["M"][g], Ms, rtol=1e-12)
        np.testing.assert_allclose(pre["b"][g], bs, rtol=1e-12)


# ============================================================================ streaming

def _stream_setup(seed=3, L=30, B=6, Rw=3, T=25):
    r = np.random.default_rng(seed)
    D, Hq, Hkv, d, dI, HI, W = 12, 4, 2, 8, 4, 4, 4
    w = dict(W_kI=r.standard_normal((dI, D)), gamma_k=np.ones(dI), W_qI=r.standard_normal((HI, dI, d)),
             gamma_q=np.ones(dI), W_g=r.standard_normal((HI, D)))
    X, Q, K, V = (r.standard_normal(s) for s in [(L, D), (W, Hq, d), (L, Hkv, d), (L, Hkv, d)])
    pre = im.prefill(X, Q, K, V, w["W_kI"], w["gamma_k"], w["W_qI"], w["gamma_q"], w["W_g"],
                     B=B, R=Rw, lam=0.9, recent_inclusive=False)
    dec = [r.standard_normal(s) for s in [(T, D), (T, Hq, d), (T, Hkv, d), (T, Hkv, d)]]
    return w, pre, dec, r.standard_normal((Hq, d))


def test_streaming_rank1_chain_equals_closed_form_and_brute_argmin():
    w, pre, (xs, qs, ks, vs), wg = _stream_setup()
    L, B, Rw = 30, 6, 3
    st_ = sm.from_prefill(pre, L, Rw)
    M0, b0 = st_.M.copy(), st_.b.copy()
    Kpool = {int(p): np.array(pre["Kc"][:, s]) for s, p in enumerate(pre["idx"])}
    Vpool = {int(p): np.array(pre["Vc"][:, s]) for s, p in enumerate(pre["idx"])}
    ev_k, ev_v = [], []
    for t in range(len(xs)):
        I_before = st_.I.copy()
        pos_before = st_.slot_pos.copy()
        p = st_.next_pos
        k_new = im.indexer_keys(xs[t][None], w["W_kI"], w["gamma_k"])[0]
        qh, gt = im.indexer_queries(qs[t][None], xs[t][None], w["W_qI"], w["gamma_q"], w["W_g"])
        newsc = [sum(gt[0, h] * max(qh[0, h] @ kk / 2.0, 0) for h in range(4)) for kk in st_.k_hat]
        o, _, ev_pos, e = sm.step(st_, xs[t], qs[t], ks[t], vs[t], w["W_kI"], w["gamma_k"],
                                  w["W_qI"], w["gamma_q"], w["W_g"], wg, 0.9)
        # brute-force argmin over candidates outside the recent window
        Inew = np.maximum(I_before, newsc)
        cands = [j for j in range(B + Rw) if pos_before[j] <= p - Rw]
        assert len(cands) == B + 1
        best = min(cands, key=lambda j: (Inew[j], -pos_before[j]))
        assert e == best and ev_pos == pos_before[best]
        assert ev_pos <= p - Rw
        assert len(st_.slot_pos) == B + Rw and len(set(st_.slot_pos.tolist())) == B + Rw
        assert st_.I[e] == pytest.approx(sum(gt[0, h] * max(qh[0, h] @ k_new / 2.0, 0) for h in range(4)))
        ev_k.append(Kpool.pop(ev_pos))
        ev_v.append(Vpool.pop(ev_pos))
        Kpool[p], Vpool[p] = ks[t], vs[t]
    for g in range(2):
        M, b = im.memory_build(np.array(ev_k)[:, g], np.array(ev_v)[:, g], 0.9, M0[g], b0[g])
        np.testing.assert_allclose(st_.M[g], M, rtol=1e-12)
        np.testing.assert_allclose(st_.b[g], b, rtol=1e-12)


# ============================================================================ MomentKV

def _linearised(q, K, V):
    d = K.shape[1]
    kbar = K.mean(0)
    x = (K - kbar) @ q / math.sqrt(d)
    return ((1 + x) @ V) / np.sum(1 + x)


def test_moment_estimate_is_linearised_softmax():
    # f^_E equals sum v_i (1 + x_i) / sum (1 + x_i), x_i = q.(k_i - k_bar)/sqrt d: exact algebra
    for seed in range(5):
        r = np.random.default_rng(seed)
        n, d = int(r.integers(1, 30)), 8
        K, V, q = r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal(d)
        mom = mk.add(mk.empty(d), K, V)
        np.testing.assert_allclose(mk.evicted_estimate(q, mom, d), _linearised(q, K, V), rtol=1e-10, atol=1e-12)


def test_moment_stats_brute_force_and_additivity():
    K, V = rnd(17, 5), rnd(17, 5)
    mom = mk.add(mk.empty(5), K, V)
    kbar, vbar, St = mk.stats(mom)
    brute = sum(np.outer(V[i] - V.mean(0), K[i] - K.mean(0)) for i in range(17))
    np.testing.assert_allclose(St, brute, rtol=1e-12, atol=1e-13)
    mom2 = mk.add(mk.add(mk.empty(5), K[:6], V[:6]), K[6:], V[6:])
    for key in ("sk", "sv", "S"):
        np.testing.assert_allclose(mom2[key], mom[key], rtol=1e-13)
    assert mom2["n"] == 17


def test_moment_estimate_second_order_convergence():
    # keys k_bar + eps delta_i: error against exact softmax shrinks as O(eps^2)
    r = np.random.default_rng(7)
    d, n = 16, 40
    kbar, delta, V, q = r.standard_normal(d), r.standard_normal((n, d)), r.standard_normal((n, d)), r.standard_normal(d)
    errs = []
    epss = [0.2, 0.1, 0.05, 0.025]
    for e in epss:
        K = kbar + e * delta
        mom = mk.add(mk.empty(d), K, V)
        exact = sp_softmax(K @ q / math.sqrt(d)) @ V
        errs.append(np.linalg.norm(mk.evicted_estimate(q, mom, d) - exact))
    slope = np.polyfit(np.log(epss), np.log(errs), 1)[0]
    assert 1.8 < slope < 2.2


def test_equal_evicted_keys_give_full_attention():
    r = np.random.default_rng(9)
    d = 8
    k = r.standard_normal(d)
    Ke, Ve = np.tile(k, (7, 1)), r.standard_normal((7, d))
    Kr, Vr, q = r.standard_normal((5, d)), r.standard_normal((5, d)), r.standard_normal(d)
    mom = mk.add(mk.empty(d), Ke, Ve)
    f_R, lse_R = im.attention_state(q, Kr, Vr, 1 / math.sqrt(d))
    fh, _ = mk.mix(q, f_R, lse_R, mom, d)
    full = sp_softmax(np.vstack([Kr, Ke]) @ q / math.sqrt(d)) @ np.vstack([Vr, Ve])
    np.testing.assert_allclose(fh, full, rtol=1e-12, atol=1e-13)


@settings(max_examples=50, deadline=None)
@given(n=st.integers(1, 20), seed=st.integers(0, 10 ** 6), sc=st.floats(0.1, 5.0))
def test_jensen_bound_holds(n, seed, sc):
    r = np.random.default_rng(seed)
    d = 6
    K, q = r.standard_normal((n, d)) * sc, r.standard_normal(d)
    mom = mk.add(mk.empty(d), K, np.zeros((n, d)))
    Z = np.sum(np.exp(K @ q / math.sqrt(d)))
    assert math.exp(mk.log_Z_hat(q, mom, d)) <= Z * (1 + 1e-12)


def test_residual_is_value_minus_estimate_at_its_key():
    # r_j = v_j - f^_E(k_j): the part-3 residual is the part-2 estimate queried with k_j
    r = np.random.default_rng(5)
    d = 8
    mom = mk.add(mk.empty(d), r.standard_normal((9, d)), r.standard_normal((9, d)))
    k, v = r.standard_normal((4, d)), r.standard_normal((4, d))
    want = np.stack([v[j] - mk.evicted_estimate(k[j], mom, d) for j in range(4)])
    np.testing.assert_allclose(mk.residual(k, v, mom, d), want, rtol=1e-12, atol=1e-13)


def test_mix_without_evictions_is_retained_output():
    f, w = mk.mix(rnd(4), np.arange(4.0), 0.3, mk.empty(4), 4)
    assert w == 1.0 and np.array_equal(f, np.arange(4.0))


def test_alpha_is_mean_of_causal_softmax_rows():
    W, Hq, Hkv, d, L = 3, 4, 2, 8, 10
    Q, K = rnd(W, Hq, d), rnd(L, Hkv, d)
    qpos = np.arange(L - W, L)
    al = mk.alpha(Q, K, qpos, 0.35, 2)
    np.testing.assert_allclose(al.sum(1), 1.0, rtol=1e-13)
    for g in range(Hkv):
        want = np.zeros(L)
        for s in range(W):
            for h in (2 * g, 2 * g + 1):
                want[:qpos[s] + 1] += sp_softmax(0.35 * K[:qpos[s] + 1, g] @ Q[s, h])
        np.testing.assert_allclose(al[g], want / 6, rtol=1e-12)
    al1 = mk.alpha(Q[-1:, :1], K[:, :1], [L - 1], 0.35, 1)
    np.testing.assert_allclose(al1[0], sp_softmax(0.35 * K[:, 0] @ Q[-1, 0]), rtol=1e-12)


def test_moment_rounds():
    r = np.random.default_rng(11)
    W, Hq, Hkv, d, L, B = 4, 4, 2, 8, 37, 5
    Q, K, V = r.standard_normal((W, Hq, d)), r.standard_normal((L, Hkv, d)), r.standard_normal((L, Hkv, d))
    out = mk.prefill(Q, K, V, B)
    assert mk.n_rounds(32768, 128) == 8 and mk.n_rounds(32768, 1024) == 5 and mk.n_rounds(37, 5) == 3
    for g in range(Hkv):
        hd = out["heads"][g]
        assert len(hd["kept"]) == B and len(hd["rounds"]) == 3
        sizes = [len(rd["pos"]) for rd in hd["rounds"]]
        assert sizes == [37, 19, 10]
        # first round: nothing evicted yet, the score is alpha * ||v||
        rd0 = hd["rounds"][0]
        np.testing.assert_allclose(rd0["scores"], out["alpha"][g] * np.linalg.norm(V[:, g], axis=1), rtol=1e-13)
        ev = np.concatenate([rd["evicted"] for rd in hd["rounds"]])
        assert hd["mom"]["n"] == L - B == len(ev)
        np.testing.assert_allclose(hd["mom"]["S"], V[ev, g].T @ K[ev, g], rtol=1e-12)
        assert sorted(np.concatenate([ev, hd["kept"]]).tolist()) == list(range(L))


# ============================================================================ MomentKV during decode

def _mstate(P, H_kv, d, L, R, seed, n_ev=0):
    """A pool of P tokens per KV head at distinct positions below L, with moments of n_ev
    evicted rows, plus the evicted rows themselves."""
    r = np.random.default_rng(seed)
    pos = np.stack([np.sort(r.choice(L, P, replace=False)) for _ in range(H_kv)])
    Kc, Vc = r.standard_normal((H_kv, P, d)), r.standard_normal((H_kv, P, d))
    ev = [(r.standard_normal((n_ev, d)), r.standard_normal((n_ev, d))) for _ in range(H_kv)]
    moms = [mk.add(mk.empty(d), k, v) if n_ev else mk.empty(d) for k, v in ev]
    return ms.MomentStreamState(pos, Kc, Vc, moms, L, R), ev


def test_stream_alpha_is_textbook_softmax_and_window_of_one():
    # catches: the new token left out of the softmax, heads summed instead of averaged
    r = np.random.default_rng(5)
    G, d, P = 3, 8, 11
    q, Kp, kn = r.standard_normal((G, d)), r.standard_normal((P, d)), r.standard_normal(d)
    al = ms.step_alpha(q, Kp, kn, 0.3)
    keys = np.vstack([Kp, kn])
    want = np.mean([sp_softmax(0.3 * keys @ qh)[:-1] for qh in q], axis=0)
    np.testing.assert_allclose(al, want, rtol=1e-13)
    # the prefill's alpha with one window query at the new token's position
    win = mk.alpha(q[None], keys[:, None, :], [P], 0.3, G)[0]
    np.testing.assert_allclose(al, win[:-1], rtol=1e-12)
    assert 0 < al.sum() < 1


def test_stream_step_hand_example():
    # zero keys: every logit is 0, alpha = 1/5; nothing evicted yet, so score = ||v|| / 5.
    # ||v|| = 3, 1, 2, 1 at positions 0..3: positions 1 and 3 tie at the lowest score and
    # the higher one (3) goes.  Output: uniform average of the pool (lse = log 4) mixed with
    # the evicted row: w_R = sigmoid(log 4 - log 1) = 4/5.
    # catches: evicting the highest score, ties evicting the lower position, folding the
    # new token into the moments, mixing with the wrong weight
    V = np.array([[3.0, 0.0], [0.0, 1.0], [0.0, 2.0], [1.0, 0.0]])
    st_ = ms.MomentStreamState([[0, 1, 2, 3]], np.zeros((1, 4, 2)), V[None], [mk.empty(2)], 4, 0)
    o, lse, slots, evp, sc = ms.step(st_, np.array([[1.0, -1.0]]), np.zeros((1, 2)), np.array([[4.0, 4.0]]))
    np.testing.assert_allclose(sc[0], [0.6, 0.2, 0.4, 0.2], rtol=1e-14)
    assert slots.tolist() == [3] and evp.tolist() == [3]
    assert st_.slot_pos.tolist() == [[0, 1, 2, 4]] and st_.next_pos == 5
    m = st_.moms[0]
    assert m["n"] == 1 and np.array_equal(m["sv"], [1.0, 0.0]) and not m["sk"].any() and not m["S"].any()
    assert lse[0] == pytest.approx(math.log(4))
    np.testing.assert_allclose(o[0], [0.8 * 1.75 + 0.2, 0.8 * 1.75], rtol=1e-14)
    # a recent window of 2 protects positions > 2: the lowest candidate is position 1
    st2 = ms.MomentStreamState([[0, 1, 2, 3]], np.zeros((1, 4, 2)), V[None], [mk.empty(2)], 4, 2)
    _, _, slots2, evp2, _ = ms.step(st2, np.array([[1.0, -1.0]]), np.zeros((1, 2)), np.array([[4.0, 4.0]]))
    assert slots2.tolist() == [1] and evp2.tolist() == [1]


def test_stream_steps_brute_force_choice_and_moments():
    # every step's choice against a from-scratch score (alpha by softmax, the covariance
    # as the centred sum over the evicted rows themselves), and the running moments
    # against the plain sums of everything evicted
    # catches: a wrong residual sign or scale, a stale moment, a candidate inside the window
    H_q, H_kv, d, P, L, R, T = 4, 2, 6, 9, 40, 3, 12
    st_, ev0 = _mstate(P, H_kv, d, L, R, seed=21, n_ev=5)
    r = np.random.default_rng(22)
    evicted = [[(k, v) for k, v in zip(*ev0[g])] for g in range(H_kv)]
    for t in range(T):
        q, kn, vn = r.standard_normal((H_q, d)), r.standard_normal((H_kv, d)), r.standard_normal((H_kv, d))
        p = st_.next_pos
        pos0, K0, V0 = st_.slot_pos.copy(), st_.Kc.copy(), st_.Vc.copy()
        o, lse, slots, evp, _ = ms.step(st_, q, kn, vn)
        for g in range(H_kv):
            Ke = np.array([k for k, _ in evicted[g]])
            Ve = np.array([v for _, v in evicted[g]])
            n = len(Ke)
            kbar, vbar = Ke.mean(0), Ve.mean(0)
            Sc = sum(np.outer(v - vbar, k - kbar) for k, v in zip(Ke, Ve))
            sc = []
            for j in range(P):
                keys = np.vstack([K0[g], kn[g]])
                al = np.mean([sp_softmax(keys @ q[h] / math.sqrt(d))[j] for h in (2 * g, 2 * g + 1)])
                rj = V0[g, j] - vbar - Sc @ K0[g, j] / (n * math.sqrt(d))
                sc.append(al * np.linalg.norm(rj))
            cands = [j for j in range(P) if pos0[g, j] <= p - R]
            best = min(cands, key=lambda j: (sc[j], -pos0[g, j]))
            assert slots[g] == best and evp[g] == pos0[g, best]
            evicted[g].append((K0[g, best], V0[g, best]))
            Ke = np.array([k for k, _ in evicted[g]])
            Ve = np.array([v for _, v in evicted[g]])
            m = st_.moms[g]
            assert m["n"] == len(Ke)
            np.testing.assert_allclose(m["sk"], Ke.sum(0), rtol=1e-12)
            np.testing.assert_allclose(m["sv"], Ve.sum(0), rtol=1e-12)
            S_ref = sum(np.outer(v, k) for k, v in zip(Ke, Ve))
            np.testing.assert_allclose(m["S"], S_ref, rtol=1e-12, atol=1e-13 * np.abs(S_ref).max())
            assert sorted(st_.slot_pos[g].tolist()) == sorted(set(pos0[g].tolist()) - {evp[g]} | {p})
            assert np.array_equal(st_.Kc[g, best], kn[g]) and np.array_equal(st_.Vc[g, best], vn[g])
            # the output: the post-hand-over pool mixed with the estimate of every row
            # evicted so far, this step's included (Jensen weight, plain loops)
            Ks = [kn[g] if j == best else K0[g, j] for j in range(P)]
            Vs = [vn[g] if j == best else V0[g, j] for j in range(P)]
            ne = len(Ke)
            kb, vb, St = _moments_s(Ke, Ve)
            for h in (2 * g, 2 * g + 1):
                fR, lz = _attend_s(q[h], Ks, Vs, 1 / math.sqrt(d))
                ZE = ne * math.exp(_dot_s(q[h], kb) / math.sqrt(d))
                wR = math.exp(lz) / (math.exp(lz) + ZE)
                fE = [vb[a] + _dot_s(St[a], q[h]) / (ne * math.sqrt(d)) for a in range(d)]
                np.testing.assert_allclose(o[h], [wR * fR[a] + (1 - wR) * fE[a] for a in range(d)],
                                           rtol=1e-10, atol=1e-12)
                assert lse[h] == pytest.approx(lz, rel=1e-12)


# ============================================================================ read-out projection

def test_memory_query_projection_special_cases():
    # catches: the projection transposed, applied after phi, or fed to the gate
    r = np.random.default_rng(31)
    H_q, H_kv, d = 4, 2, 5
    q, w_g = r.standard_normal((H_q, d)), r.standard_normal((H_q, d))
    M, b = r.standard_normal((H_kv, d, d)), np.abs(r.standard_normal((H_kv, d))) + 0.5
    base_m, base_g = im.memory_readout(q, M, b, w_g)
    # identity: the plain read-out
    m, g = im.memory_readout(q, M, b, w_g, q_mem=im.memory_query(q, np.eye(d)))
    np.testing.assert_allclose(m, base_m, rtol=1e-14)
    assert np.array_equal(g, base_g)
    # permutation P: phi(Pq) = P phi(q), so reading with P equals reading M P and P^T b
    perm = np.array([2, 0, 4, 1, 3])
    P = np.eye(d)[perm]
    assert not np.array_equal(P, P.T)
    m, g = im.memory_readout(q, M, b, w_g, q_mem=im.memory_query(q, P))
    m2, _ = im.memory_readout(q, M @ P, np.einsum("ij,gi->gj", P, b), w_g)
    np.testing.assert_allclose(m, m2, rtol=1e-13)
    assert np.array_equal(g, base_g)
    # zero projection: phi(0) = 1, so m = M 1 / (b . 1 + eps) for every query; the gate
    # still follows the model query
    m, g = im.memory_readout(q, M, b, w_g, q_mem=im.memory_query(q, np.zeros((d, d))))
    for h in range(H_q):
        np.testing.assert_allclose(m[h], M[h // 2].sum(1) / (b[h // 2].sum() + 1e-6), rtol=1e-13)
    assert np.array_equal(g, base_g)
    # W = -I: phi acts on the projected query (phi(-q) differs from -phi(q))
    m, _ = im.memory_readout(q, M, b, w_g, q_mem=im.memory_query(q, -np.eye(d)))
    for h in range(H_q):
        f = np.where(-q[h] > 0, -q[h] + 1.0, np.exp(-q[h]))
        np.testing.assert_allclose(m[h], M[h // 2] @ f / (b[h // 2] @ f + 1e-6), rtol=1e-13)


# ============================================================================ attention-state memory

def test_asm_own_state_restores_full_attention():
    # a query whose retrieved state is its own prefix state recovers attention over the
    # prefix and the local tokens together (the online-softmax identity); a one-member
    # cluster keeps its member's state exactly
    # catches: a wrong merge weight, a dropped partition, an unscaled logit
    r = np.random.default_rng(41)
    N, H_q, H_kv, d, L, Lloc = 5, 4, 2, 8, 30, 7
    Q = r.standard_normal((N, H_q, d))
    K, V = r.standard_normal((L, H_kv, d)), r.standard_normal((L, H_kv, d))
    Kl, Vl = r.standard_normal((Lloc, H_kv, d)), r.standard_normal((Lloc, H_kv, d))
    sc = 1 / math.sqrt(d)
    a, lse = asm.prefix_states(Q, K, V, sc)
    for h in range(H_q):
        g = h // 2
        C = Q[:, h]                       # every query its own centroid
        a_bar, lse_bar = asm.aggregate(a[:, h], lse[:, h], np.arange(N), N)
        np.testing.assert_array_equal(a_bar, a[:, h])
        np.testing.assert_array_equal(lse_bar, lse[:, h])
        for i in range(N):
            a_loc, l_loc = im.attention_state(Q[i, h], Kl[:, g], Vl[:, g], sc)
            (o, l), k = asm.output(Q[i, h], C, a_bar, lse_bar, a_loc, l_loc)
            assert k == i
            keys, vals = np.vstack([K[:, g], Kl[:, g]]), np.vstack([V[:, g], Vl[:, g]])
            w = sp_softmax(sc * keys @ Q[i, h])
            np.testing.assert_allclose(o, w @ vals, rtol=1e-12)
            assert l == pytest.approx(sp_lse(sc * keys @ Q[i, h]), rel=1e-13)


def test_asm_aggregate_is_partition_weighted_mean():
    # catches: an unweighted mean of the outputs, the summed (not mean) partition
    r = np.random.default_rng(42)
    N, d, K = 12, 6, 4
    a, lse = r.standard_normal((N, d)), r.standard_normal(N) * 3
    idx = np.array([0, 1, 1, 2, 0, 0, 1, 2, 2, 2, 0, 1])     # cluster 3 stays empty
    a_bar, lse_bar = asm.aggregate(a, lse, idx, K)
    for k in range(3):
        m = idx == k
        Z = np.exp(lse[m])
        np.testing.assert_allclose(a_bar[k], (Z[:, None] * a[m]).sum(0) / Z.sum(), rtol=1e-12)
        assert lse_bar[k] == pytest.approx(math.log(Z.mean()), rel=1e-12)
    assert lse_bar[3] == -np.inf and not a_bar[3].any()
    # identical members: the cluster's state is the member's
    a2, l2 = asm.aggregate(np.tile(a[:1], (5, 1)), np.full(5, lse[0]), np.zeros(5, int), 1)
    np.testing.assert_allclose(a2[0], a[0], rtol=1e-14)
    assert l2[0] == pytest.approx(lse[0], rel=1e-14)


def test_kmeans_lloyd_steps():
    # catches: argmax instead of argmin, ties to the higher index, an empty cluster moved
    r = np.random.default_rng(43)
    centers = np.array([[10.0, 0, 0], [0, 10.0, 0], [0, 0, 10.0]])
    X = np.vstack([c + 0.1 * r.standard_normal((20, 3)) for c in centers])
    C0 = np.vstack([X[0], X[20], X[40], [100.0, 100, 100]])   # the last seed draws nobody
    C, idx = asm.kmeans(X, C0, 3)
    assert np.array_equal(idx, np.repeat([0, 1, 2], 20))
    for k in range(3):
        np.testing.assert_allclose(C[k], X[20 * k:20 * (k + 1)].mean(0), rtol=1e-13)
    assert np.array_equal(C[3], [100.0, 100, 100])
    # brute-force assignment and a tie between two equal centroids
    Y = r.standard_normal((15, 3))
    Cb = r.standard_normal((5, 3))
    Cb[3] = Cb[1]
    got, d2 = asm.kmeans_assign(Y, Cb)
    for i in range(15):
        dist = [float(((Y[i] - c) ** 2).sum()) for c in Cb]
        assert got[i] == min(range(5), key=lambda k: (dist[k], k))
        assert got[i] != 3
    # Lloyd never increases the within-cluster sum of squares
    Cc, last = Cb.copy(), None
    for _ in range(5):
        idx = asm.kmeans_assign(Y, Cc)[0]
        inertia = sum(((Y[i] - Cc[idx[i]]) ** 2).sum() for i in range(15))
        assert last is None or inertia <= last + 1e-12
        last = inertia
        Cc = asm.kmeans_update(Y, idx, Cc)


def test_asm_lookup_is_cosine_argmax():
    # catches: a plain dot product (sensitive to the centroid's norm)
    r = np.random.default_rng(44)
    C = r.standard_normal((9, 5))
    for _ in range(20):
        q = r.standard_normal(5)
        k = asm.lookup(q, C)
        cos = [float(c @ q / np.linalg.norm(c) / np.linalg.norm(q)) for c in C]
        assert k == max(range(9), key=lambda j: (cos[j], -j))
        assert asm.lookup(3.7 * q, C) == k
        C2 = C.copy()
        C2[k] *= 0.01                     # a short centroid in the same direction still wins
        assert asm.lookup(q, C2) == k


# ============================================================================ chunked pre-eviction

def _chunk_setup(L, seed, D=24, H_q=4, H_kv=2, d=8, H_I=3, d_I=6):
    r = np.random.default_rng(seed)
    return dict(X=r.standard_normal((L, D)), Q=r.standard_normal((L, H_q, d)),
                K=r.standard_normal((L, H_kv, d)), V=r.standard_normal((L, H_kv, d)),
                W_kI=r.standard_normal((d_I, D)) / math.sqrt(D), gamma_k=1 + 0.1 * r.standard_normal(d_I),
                W_qI=r.standard_normal((H_I, d_I, d)) / math.sqrt(d), gamma_q=1 + 0.1 * r.standard_normal(d_I),
                W_g=r.standard_normal((H_I, D)) / math.sqrt(D))


def _chunked(c, B, R, lam, C, W):
    return ck.prefill_chunked(c["X"], c["Q"], c["K"], c["V"], c["W_kI"], c["gamma_k"], c["W_qI"], c["gamma_q"],
                              c["W_g"], B, R, lam, C, W)


def test_chunked_single_chunk_is_one_shot_prefill():
    # catches: a chunk schedule that changes the one-shot selection, a wrong window
    L, W, B, R, lam = 40, 6, 12, 3, 0.9
    c = _chunk_setup(L, 51)
    out = _chunked(c, B, R, lam, L, W)
    pre = im.prefill(c["X"], c["Q"][L - W:], c["K"], c["V"], c["W_kI"], c["gamma_k"], c["W_qI"], c["gamma_q"],
                     c["W_g"], B, R, lam)
    assert np.array_equal(out["pos"], pre["idx"])
    np.testing.assert_allclose(out["I"], pre["I"][pre["idx"]], rtol=1e-13)
    np.testing.assert_allclose(out["k_hat"], pre["k_hat"][pre["idx"]], rtol=1e-13)
    np.testing.assert_allclose(out["M"], pre["M"], rtol=1e-12)
    np.testing.assert_allclose(out["b"], pre["b"], rtol=1e-12)
    np.testing.assert_array_equal(out["K"], c["K"][pre["idx"]])


def test_chunked_running_max_budget_and_fold_composition():
    # catches: a pooled key losing its earlier importance, the window taken at the chunk's
    # start, a candidate from the recent window evicted, a fold in the wrong order
    L, C, W, B, R, lam = 53, 12, 5, 10, 3, 0.8
    c = _chunk_setup(L, 52)
    out = _chunked(c, B, R, lam, C, W)
    ends = [min(L, s + C) for s in range(0, L, C)]
    kh = im.indexer_keys(c["X"], c["W_kI"], c["gamma_k"])
    windows = []
    for e in ends:
        qh, gt = im.indexer_queries(c["Q"][e - W:e], c["X"][e - W:e], c["W_qI"], c["gamma_q"], c["W_g"])
        windows.append((e, qh, gt))
    seen, evicted_all = 0, []
    prev = np.zeros(0, np.int64)
    for (e, _, _), st in zip(windows, out["steps"]):
        assert len(st["kept"]) == min(B, e) and np.all(np.diff(st["kept"]) > 0)
        assert set(range(e - R, e)) <= set(st["kept"].tolist())
        assert sorted(st["kept"].tolist() + st["evicted"].tolist()) == sorted(prev.tolist() + list(range(seen, e)))
        evicted_all += st["evicted"].tolist()
        prev, seen = st["kept"], e
    # every pooled key's importance: the max over each later window (the one of its own
    # chunk only from queries at or after it)
    for t, It in zip(out["pos"], out["I"]):
        best = -np.inf
        for e, qh, gt in windows:
            if e <= t:
                continue
            for i in range(W):
                if e - W + i >= t:
                    best = max(best, sum(gt[i, h] * max(qh[i, h] @ kh[t] / math.sqrt(kh.shape[1]), 0.0)
                                         for h in range(qh.shape[1])))
        assert It == pytest.approx(best, rel=1e-12)
    # the per-chunk folds compose into one fold over all evictions in eviction order
    for g in range(2):
        Mr, br = im.memory_build(c["K"][evicted_all, g], c["V"][evicted_all, g], lam)
        np.testing.assert_allclose(out["M"][g], Mr, rtol=1e-12)
        np.testing.assert_allclose(out["b"][g], br, rtol=1e-12)


# ============================================================================ compositions, by brute force
#
# Each pipeline function below is checked end to end against the definitions written out
# as plain loops over scalars: no oracle helper other than the function under test takes
# part in the expected value.

def _phi_s(x):
    return x + 1.0 if x > 0 else math.exp(x)


def _sig_s(x):
    return 1.0 / (1.0 + math.exp(-x))


def _dot_s(a, b):
    return sum(float(x) * float(y) for x, y in zip(a, b))


def _attend_s(q, Ks, Vs, scale):
    """Plain softmax attention of one query over a list of rows: output and log Z."""
    s = [scale * _dot_s(q, k) for k in Ks]
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    Z = sum(e)
    out = np.array([sum(e[j] * float(Vs[j][i]) for j in range(len(Ks))) / Z for i in range(len(q))])
    return out, mx + math.log(Z)


def _moments_s(Ke, Ve):
    """Key mean, value mean and sum_i (v_i - v_bar)(k_i - k_bar)^T over evicted rows."""
    n, d = len(Ke), len(Ke[0])
    kbar = [sum(float(Ke[i][c]) for i in range(n)) / n for c in range(d)]
    vbar = [sum(float(Ve[i][c]) for i in range(n)) / n for c in range(d)]
    St = [[sum((float(Ve[i][a]) - vbar[a]) * (float(Ke[i][c]) - kbar[c]) for i in range(n))
           for c in range(d)] for a in range(d)]
    return kbar, vbar, St


def _alpha_s(Q, K, g, G, q_pos, scale):
    """alpha_j of KV head g: causal softmax weight of key j, averaged over window queries
    and the G query heads of the group."""
    W, L = Q.shape[0], K.shape[0]
    al = [0.0] * L
    for s in range(W):
        for h in range(g * G, (g + 1) * G):
            n = int(q_pos[s]) + 1
            lg = [scale * _dot_s(Q[s, h], K[j, g]) for j in range(n)]
            mx = max(lg)
            e = [math.exp(x - mx) for x in lg]
            Z = sum(e)
            for j in range(n):
                al[j] += e[j] / Z
    return [a / (W * G) for a in al]


def test_moment_rounds_selection_and_residuals_brute_force():
    # Every round of the moment-informed prefill: the round's scores equal
    # alpha_j * ||v_j - v_bar - S~ k_j / (n_e sqrt d)|| with the moments of every token
    # evicted in EARLIER rounds (r_j = v_j before any eviction), the round keeps
    # max(B, ceil(n/2)) tokens, and every kept score beats every evicted one (equal
    # scores: the lower position is kept).
    # catches: keeping the lowest scores; later rounds scored with empty or stale moments.
    r = np.random.default_rng(21)
    W, Hq, Hkv, d, L, B = 3, 4, 2, 6, 41, 5
    Q, K, V = r.standard_normal((W, Hq, d)), r.standard_normal((L, Hkv, d)), r.standard_normal((L, Hkv, d))
    out = mk.prefill(Q, K, V, B)
    G, scale = Hq // Hkv, 1 / math.sqrt(d)
    q_pos = list(range(L - W, L))
    for g in range(Hkv):
        al = _alpha_s(Q, K, g, G, q_pos, scale)
        hd = out["heads"][g]
        pos = list(range(L))
        evicted = []
        assert len(hd["rounds"]) == 4          # 41 -> 21 -> 11 -> 6 -> 5
        for rd in hd["rounds"]:
            assert rd["pos"].tolist() == pos
            if evicted:
                n_e = len(evicted)
                kbar, vbar, St = _moments_s([K[e, g] for e in evicted], [V[e, g] for e in evicted])
            want = []
            for j in pos:
                if not evicted:
                    res = [float(x) for x in V[j, g]]
                else:
                    res = [float(V[j, g][a]) - vbar[a] - _dot_s(St[a], K[j, g]) / (n_e * math.sqrt(d))
                           for a in range(d)]
                want.append(al[j] * math.sqrt(sum(x * x for x in res)))
            np.testing.assert_allclose(rd["scores"], want, rtol=1e-10)
            keep_n = max(B, -(-len(pos) // 2))
            kept, ev = rd["kept"].tolist(), rd["evicted"].tolist()
            assert len(kept) == keep_n and sorted(kept + ev) == pos and kept == sorted(kept)
            sc = dict(zip(pos, want))
            for a in kept:
                for e in ev:
                    assert sc[a] > sc[e] or (sc[a] == sc[e] and a < e)
            evicted += ev
            pos = kept
        assert hd["kept"].tolist() == pos and hd["mom"]["n"] == len(evicted) == L - B


@pytest.mark.parametrize("B", [5, 60])
def test_momentkv_decode_appends_then_mixes_brute_force(B):
    # Decode over each KV head's kept tokens PLUS every token appended so far, mixed with
    # the first-order estimate by the Jensen weight.  B >= L (nothing evicted) must be
    # textbook softmax attention over the whole sequence.
    # catches: attending without appending the new K/V; mixing weight or estimate slips.
    r = np.random.default_rng(22)
    W, Hq, Hkv, d, L, T = 3, 4, 2, 6, 23, 3
    Q, K, V = r.standard_normal((W, Hq, d)), r.standard_normal((L, Hkv, d)), r.standard_normal((L, Hkv, d))
    qs, ks, vs = r.standard_normal((T, Hq, d)), r.standard_normal((T, Hkv, d)), r.standard_normal((T, Hkv, d))
    heads = mk.prefill(Q, K, V, B)["heads"]
    o, lse, w = mk.decode(qs, ks, vs, K, V, heads)
    G, scale = Hq // Hkv, 1 / math.sqrt(d)
    for g in range(Hkv):
        kept = heads[g]["kept"].tolist()
        evicted = [t for t in range(L) if t not in kept]
        assert (len(evicted) == 0) == (B >= L)
        if evicted:
            kbar, vbar, St = _moments_s([K[e, g] for e in evicted], [V[e, g] for e in evicted])
        for t in range(T):
            Ks = [K[j, g] for j in kept] + [ks[u, g] for u in range(t + 1)]
            Vs = [V[j, g] for j in kept] + [vs[u, g] for u in range(t + 1)]
            for h in range(g * G, (g + 1) * G):
                fR, lseR = _attend_s(qs[t, h], Ks, Vs, scale)
                assert lse[t, h] == pytest.approx(lseR, rel=1e-12)
                if not evicted:
                    np.testing.assert_allclose(o[t, h], fR, rtol=1e-11, atol=1e-13)
                    assert w[t, h] == 1.0
                    continue
                n_e = len(evicted)
                ZE = n_e * math.exp(scale * _dot_s(qs[t, h], kbar))
                wR = math.exp(lseR) / (math.exp(lseR) + ZE)
                fE = [vbar[a] + _dot_s(St[a], qs[t, h]) / (n_e * math.sqrt(d)) for a in range(d)]
                want = [wR * fR[a] + (1 - wR) * fE[a] for a in range(d)]
                assert w[t, h] == pytest.approx(wR, rel=1e-11)
                np.testing.assert_allclose(o[t, h], want, rtol=1e-10, atol=1e-12)


def test_streaming_step_output_brute_force():
    # Each streaming step's output is plain softmax attention over the pool AFTER the
    # hand-over (the evicted slot holds the new token) plus sigmoid(w_g.q) M' phi(q) /
    # (b'.phi(q) + eps), where M' = lam M + v_e phi(k_e)^T and b' = lam b + phi(k_e) fold the
    # evicted row in first.
    # catches: reading out with the memory from before the fold; attending before the
    # hand-over; the gate or the fold applied wrongly.
    w, pre, (xs, qs, ks, vs), wg = _stream_setup(seed=8, T=12)
    Rw, lam, eps = 3, 0.9, 1e-6
    st_ = sm.from_prefill(pre, 30, Rw)
    Hkv, P, d = st_.Kc.shape
    G = qs.shape[1] // Hkv
    for t in range(len(xs)):
        Kc0, Vc0, M0, b0 = st_.Kc.copy(), st_.Vc.copy(), st_.M.copy(), st_.b.copy()
        o, lse, ev_pos, e = sm.step(st_, xs[t], qs[t], ks[t], vs[t], w["W_kI"], w["gamma_k"],
                                    w["W_qI"], w["gamma_q"], w["W_g"], wg, lam, eps_mem=eps)
        for g in range(Hkv):
            fk = [_phi_s(float(x)) for x in Kc0[g, e]]
            Mg = [[lam * M0[g][a][c] + float(Vc0[g, e][a]) * fk[c] for c in range(d)] for a in range(d)]
            bg = [lam * b0[g][c] + fk[c] for c in range(d)]
            Ks = [ks[t, g] if j == e else Kc0[g, j] for j in range(P)]
            Vs = [vs[t, g] if j == e else Vc0[g, j] for j in range(P)]
            for h in range(g * G, (g + 1) * G):
                q = qs[t, h]
                att, lz = _attend_s(q, Ks, Vs, 1 / math.sqrt(d))
                fq = [_phi_s(float(x)) for x in q]
                den = _dot_s(bg, fq) + eps
                gate = _sig_s(_dot_s(wg[h], q))
                want = [att[a] + gate * _dot_s(Mg[a], fq) / den for a in range(d)]
                np.testing.assert_allclose(o[h], want, rtol=1e-10, atol=1e-12)
                assert lse[h] == pytest.approx(lz, rel=1e-12)


def test_indexmem_decode_with_memory_brute_force():
    # Decode with a non-zero memory: o = softmax attention over the retained slots plus the
    # appended ones, plus sigmoid(w_g.q) M phi(q) / (b.phi(q) + eps), with M, b held fixed.
    # catches: the gate dropped (the only other end-to-end pin has M = 0).
    r = np.random.default_rng(23)
    Hq, Hkv, d, n0, T, lam, eps = 4, 2, 6, 7, 3, 0.8, 1e-6
    cap = n0 + T
    Kc, Vc = np.zeros((Hkv, cap, d)), np.zeros((Hkv, cap, d))
    Kc[:, :n0], Vc[:, :n0] = r.standard_normal((Hkv, n0, d)), r.standard_normal((Hkv, n0, d))
    # the memory of 9 evicted rows per KV head, folded one at a time
    M, b = np.zeros((Hkv, d, d)), np.zeros((Hkv, d))
    for g in range(Hkv):
        for _ in range(9):
            k, v = r.standard_normal(d), r.standard_normal(d)
            for a in range(d):
                for c in range(d):
                    M[g, a, c] = lam * M[g, a, c] + v[a] * _phi_s(k[c])
            for c in range(d):
                b[g, c] = lam * b[g, c] + _phi_s(k[c])
    qs, ks, vs = r.standard_normal((T, Hq, d)), r.standard_normal((T, Hkv, d)), r.standard_normal((T, Hkv, d))
    wg = r.standard_normal((Hq, d))
    o, lse, _, _ = im.decode(qs, ks, vs, Kc, Vc, n0, M, b, wg, eps=eps)
    G = Hq // Hkv
    for t in range(T):
        for h in range(Hq):
            g, q = h // G, qs[t, h]
            Ks = [Kc[g, j] for j in range(n0)] + [ks[u, g] for u in range(t + 1)]
            Vs = [Vc[g, j] for j in range(n0)] + [vs[u, g] for u in range(t + 1)]
            att, lz = _attend_s(q, Ks, Vs, 1 / math.sqrt(d))
            fq = [_phi_s(float(x)) for x in q]
            gate = _sig_s(_dot_s(wg[h], q))
            want = [att[a] + gate * _dot_s(M[g, a], fq) / (_dot_s(b[g], fq) + eps) for a in range(d)]
            np.testing.assert_allclose(o[t, h], want, rtol=1e-10, atol=1e-12)
            assert lse[t, h] == pytest.approx(lz, rel=1e-12)
