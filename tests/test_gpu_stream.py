"""kvm_stream_evict + kvm_decode_attn_mem(append_slot) against the streaming oracle, step
by step, from a pool built by the oracle's prefill (the device state starts from the same
values, rounded to the storage precision).

Decision rule: the evicted slot must equal the oracle's, decided on the oracle's
importances rounded to fp32 (the kernel's precision), unless the two candidates' scores
lie within 1e-5 of each other; after such a near-tie the two states legitimately diverge,
so the comparison stops there, after at least 8 compared steps."""
import numpy as np
import pytest

from oracle import indexmem as im
from oracle import streaming as so
from synth import WORKLOADS, gen

pytestmark = pytest.mark.gpu

CASES = [
    # workload, overrides, steps, batch elements
    ("llama8b_layer_131k_stream", dict(L=1024, B=120, R=64), 48, 1),
    ("llama8b_layer_131k_stream", dict(L=700, B=33, R=17, W=32, needles=0), 40, 2),
    ("tiny_fp32", dict(streaming=True, B=40, R=8, recent_inclusive=False), 40, 1),
    # the timed pool: 1024 + 64 slots (68 score blocks of 16 keys), shorter prefill
    ("llama8b_layer_131k_stream", dict(L=2048, B=1024, R=64), 16, 1),
]


@pytest.mark.parametrize("wl,over,steps,nb", CASES)
def test_stream_steps_match_oracle(wl, over, steps, nb):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise, assert_output

    cfg = WORKLOADS[wl].with_(**over)
    dt = cfg.dtype
    lam = float(np.float32(cfg.lam))
    bl = list(range(nb))
    p = gen.make_prefill(cfg, batches=bl)
    dec = gen.make_decode(cfg, batches=bl, steps=steps)
    f = lambda x: gen.from_storage(x, dt)
    W_kI, W_qI, W_g, w_g = f(p["W_kI"]), f(p["W_qI"]), f(p["W_g"]), f(p["w_g"])
    pres = [im.prefill(f(p["X"][i]), f(p["Qwin"][i]), f(p["K"][i]), f(p["V"][i]), W_kI, p["gamma_k"], W_qI,
                       p["gamma_q"], W_g, cfg.B, cfg.R, lam, cfg.recent_inclusive, eps=cfg.eps_rms) for i in bl]
    P = len(pres[0]["idx"])
    cap = api.cache_cap(P)
    sts = [so.from_prefill(pre, cfg.L, cfg.R) for pre in pres]

    # device state (storage precision)
    Kc = np.zeros((nb, cfg.H_kv, cap, cfg.d))
    Vc = np.zeros((nb, cfg.H_kv, cap, cfg.d))
    for i, pre in enumerate(pres):
        Kc[i, :, :P] = pre["Kc"][:, :P]
        Vc[i, :, :P] = pre["Vc"][:, :P]
    dKc = to_dev(gen.to_storage(Kc, dt))
    dVc = to_dev(gen.to_storage(np.ascontiguousarray(Vc.transpose(0, 1, 3, 2)), dt))
    dM = to_dev(np.stack([pre["M"] for pre in pres]).astype(np.float32))
    db = to_dev(np.stack([pre["b"] for pre in pres]).astype(np.float32))
    khat = to_dev(np.stack([pre["k_hat"][pre["idx"]] for pre in pres]).astype(np.float32))
    Ipool = to_dev(np.stack([pre["I"][pre["idx"]] for pre in pres]).astype(np.float32))
    spos = to_dev(np.stack([pre["idx"] for pre in pres]).astype(np.int32))
    npos = to_dev(np.full(nb, cfg.L, np.int32))
    lens = to_dev(np.full(nb, P, np.int32))
    wts = [to_dev(p[k]) for k in ("W_kI", "gamma_k", "W_qI", "gamma_q", "W_g")]
    dwg = to_dev(p["w_g"])

    live = [True] * nb
    compared = [0] * nb
    for t in range(steps):
        x_t, q_t = dec["x_new"][t], dec["q"][t]
        k_t, v_t = dec["k_new"][t], dec["v_new"][t]
        e_dev = api.kvm_stream_evict(to_dev(x_t), to_dev(q_t), *wts, khat, Ipool, spos, npos, dKc, dVc, dM, db,
                                     lam, cfg.R, eps=cfg.eps_rms)
        o = api.kvm_decode_attn_mem(to_dev(q_t), dKc, dVc, lens, k_new=to_dev(k_t), v_new=to_dev(v_t),
                                    append_slot=e_dev, M=dM, bvec=db, w_g=dwg)
        torch.cuda.synchronize()
        g_e, g_pos, g_I, g_k = to_np(e_dev), to_np(spos), to_np(Ipool), to_np(khat)
        g_M, g_b, g_o = to_np(dM), to_np(db), to_np(o)
        for i in bl:
            if not live[i]:
                continue
            st = sts[i]
            # the oracle's importances after this step's max-update, before the slot hand-over
            q_hat, gate = im.indexer_queries(f(q_t)[i:i + 1], f(x_t)[i:i + 1], W_qI, p["gamma_q"], W_g, cfg.eps_rms)
            I_upd = np.maximum(st.I, so.new_query_scores(q_hat[0], gate[0], st.k_hat))
            pos_before = st.slot_pos.copy()
            o_ref, _, ev_pos, e_ref = so.step(st, f(x_t[i]), f(q_t[i]), f(k_t[i]), f(v_t[i]), W_kI, p["gamma_k"],
                                              W_qI, p["gamma_q"], W_g, w_g, lam, cfg.eps_rms)
            e_got = int(g_e[i])
            if e_got != e_ref:
                # a near-tie in the kernel's precision ends this sequence's comparison: both
                # slots must be candidates whose fp32 importances agree to 1e-5
                p_now = cfg.L + t
                assert pos_before[e_got] <= p_now - cfg.R, f"step {t}: slot {e_got} is in the recent window"
                a32, b32 = float(np.float32(I_upd[e_got])), float(np.float32(I_upd[e_ref]))
                assert abs(a32 - b32) <= 1e-5 * abs(b32), \
                    f"seq {i} step {t}: evicted slot {e_got} (I={a32}) != oracle {e_ref} (I={b32})"
                assert compared[i] >= min(8, steps), f"seq {i} step {t}: near-tie after {compared[i]} steps"
                live[i] = False
                continue
            assert int(g_pos[i][e_got]) == cfg.L + t
            np.testing.assert_array_equal(g_pos[i], st.slot_pos)
            assert normwise(g_I[i], st.I) < 1e-5, f"seq {i} step {t}: importances"
            assert normwise(g_k[i], st.k_hat) < 1e-5, f"seq {i} step {t}: pooled indexer keys"
            assert normwise(g_M[i], st.M) < 1e-5, f"seq {i} step {t}: M"
            assert normwise(g_b[i], st.b) < 1e-5, f"seq {i} step {t}: b"
            assert_output(g_o[i], o_ref, dt, f"seq {i} step {t}: o")
            np.testing.assert_allclose(g_o[i], o_ref, rtol=2e-4, atol=2e-4 * np.abs(o_ref).max())
            compared[i] += 1
    assert min(compared) >= min(8, steps)
