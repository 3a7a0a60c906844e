"""The oracle against hand-derived fixtures (tests/golden/*.json)."""
import json
import math
import os

import numpy as np

from oracle import indexmem as im
from oracle import momentkv as mk

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def arr(x):
    return np.array([[float(v) for v in r] if isinstance(r, list) else float(r) for r in x])


def test_indexer_tiny():
    g = load("indexer_tiny.json")
    i, e = g["inputs"], g["expected"]
    A = im.score_matrix(np.array(i["q_hat"], float), np.array(i["gate"]), np.array(i["k_hat"], float),
                        np.array(i["q_pos"]))
    np.testing.assert_allclose(A, arr(e["A"]), rtol=1e-14)
    I = im.importance(A)
    np.testing.assert_allclose(I, e["I"], rtol=1e-14)
    idx, sm = im.topk_select(I, i["B"], i["R"])
    assert idx.tolist() == e["idx"]
    assert sm.tolist() == e["slot_map"]


def test_memory_tiny():
    g = load("memory_tiny.json")
    i, e = g["inputs"], g["expected"]
    M, b = im.memory_build(np.array(i["K_ev"]), np.array(i["V_ev"]), i["lam"])
    np.testing.assert_allclose(M, e["M"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(b, e["b"], rtol=1e-14)
    q = np.array([i["q"]])
    m, gg = im.memory_readout(q, M[None], b[None], np.array([i["w_g"]]), eps=i["eps"])
    np.testing.assert_allclose(m[0], e["m"], rtol=1e-14)
    assert gg[0] == e["g"]
    a, lse = im.attention_state(q[0], np.array(i["Kc"]), np.array(i["Vc"]), 0.7)
    np.testing.assert_allclose(a, e["a"], rtol=1e-14)
    assert math.isclose(lse, e["lse"], rel_tol=1e-14)
    o = im.residual_output(a[None], m, gg)
    np.testing.assert_allclose(o[0], e["o"], rtol=1e-14)


def test_moments_tiny():
    g = load("moments_tiny.json")
    i, e = g["inputs"], g["expected"]
    mom = mk.add(mk.empty(2), np.array(i["K_ev"]), np.array(i["V_ev"]))
    assert mom["n"] == e["n"]
    np.testing.assert_allclose(mom["sk"], e["sk"])
    np.testing.assert_allclose(mom["sv"], e["sv"])
    np.testing.assert_allclose(mom["S"], e["S"])
    _, _, St = mk.stats(mom)
    np.testing.assert_allclose(St, e["S_tilde"], atol=1e-15)
    q = np.array(i["q"])
    np.testing.assert_allclose(mk.evicted_estimate(q, mom, 2), e["f_E_hat"], atol=1e-14)
    assert math.isclose(mk.log_Z_hat(q, mom, 2), e["log_Z_hat"], rel_tol=1e-14)
    Kev = np.array(i["K_ev"])
    Z = np.sum(np.exp(Kev @ q / math.sqrt(2)))
    assert math.isclose(Z, e["Z_exact"], rel_tol=1e-14)
    assert math.exp(e["log_Z_hat"]) <= Z
    r = mk.residual(np.array([i["k_j"]]), np.array([i["v_j"]]), mom, 2)[0]
    np.testing.assert_allclose(r, e["r"], atol=1e-15)
    r2 = mk.residual(np.array([i["k_j2"]]), np.array([i["v_j2"]]), mom, 2)[0]
    np.testing.assert_allclose(r2, e["r2"], atol=1e-14)
    s = mk.score(np.array([i["alpha_j"]]), np.array([i["k_j"]]), np.array([i["v_j"]]), mom, 2)[0]
    assert math.isclose(s, e["score"], rel_tol=1e-14)
    f, w = mk.mix(q, np.array(i["f_R"]), i["lse_R"], mom, 2)
    assert math.isclose(w, e["w_R"], rel_tol=1e-14)
    np.testing.assert_allclose(f, e["f_hat"], atol=1e-14)
