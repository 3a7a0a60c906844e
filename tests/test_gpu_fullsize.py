"""Full-size checks at the workloads' real shapes, in the launch configuration the
benchmark times (same entry points, cache capacity keep + 512, automatic split count).

* Llama-3.1-8B-shaped layer, batch 8, 16384-token prefill evicted to B = 1638 (R = 32
  inside): every sequence's importance I and kept set against the oracle, the caches
  bit-exact, M and b of sampled (sequence, KV head) pairs; then decode steps over the
  oracle's own prefill state uploaded at full size, every output checked.
* Streaming step at the 131072-token workload's pool size (1024 + 64 slots, D = 4096).
* MomentKV alpha at the Qwen3-4B shape (L = 32768, batch 4) for sampled pairs.
Oracle work is bounded by sampling where a full pass would take minutes."""
import math

import numpy as np
import pytest

from oracle import indexmem as im
from oracle import momentkv as mk
from oracle import streaming as so
from synth import WORKLOADS, gen

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BENCH_T = 512     # decode steps the benchmark reserves cache room for
DEC_STEPS = 3     # decode steps checked here


@pytest.fixture(scope="module")
def cfg3_layer():
    cfg = WORKLOADS["llama8b_32L_16k_b8"].with_(layers=1)
    p = gen.make_prefill(cfg)
    return cfg, p


@pytest.mark.timeout(900)
def test_cfg3_prefill_full_size(cfg3_layer):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, set_check, normwise
    cfg, p = cfg3_layer
    f = lambda x: gen.from_storage(x, cfg.dtype)
    lam = float(np.float32(cfg.lam))
    X, Kt, Vt = to_dev(p["X"]), to_dev(p["K"]), to_dev(p["V"])
    I = api.kvm_index_score(X, to_dev(p["Qwin"]), to_dev(p["W_kI"]), to_dev(p["gamma_k"]), to_dev(p["W_qI"]),
                            to_dev(p["gamma_q"]), to_dev(p["W_g"]), eps=cfg.eps_rms)
    idx, sm = api.kvm_topk_select(I, cfg.B, cfg.R, cfg.recent_inclusive)
    keep = idx.shape[1]
    cap = api.cache_cap(keep + BENCH_T)
    M = torch.zeros((cfg.b, cfg.H_kv, cfg.d, cfg.d), device="cuda")
    bv = torch.zeros((cfg.b, cfg.H_kv, cfg.d), device="cuda")
    Kc, Vc = api.kvm_compact_kv(Kt, Vt, sm, idx, keep, cap, M=M, bvec=bv, lam=lam)
    torch.cuda.synchronize()
    gI, gidx, gK, gV, gM, gb = (to_np(t) for t in (I, idx, Kc, Vc, M, bv))
    Wk, Wq, Wg = f(p["W_kI"]), f(p["W_qI"]), f(p["W_g"])
    for i in range(cfg.b):
        Xi = f(p["X"][i])
        kh = im.indexer_keys(Xi, Wk, p["gamma_k"], cfg.eps_rms)
        qh, g = im.indexer_queries(f(p["Qwin"][i]), Xi[cfg.L - cfg.W:], Wq, p["gamma_q"], Wg, cfg.eps_rms)
        Iref = im.importance(im.score_matrix(qh, g, kh, np.arange(cfg.L - cfg.W, cfg.L)))
        assert np.max(np.abs(gI[i] - Iref) / np.maximum(np.abs(Iref), 1e-3)) < 2e-6, f"seq {i}: I"
        n_diff = set_check(gidx[i], Iref, cfg.B, cfg.R, cfg.recent_inclusive)
        # the caches hold exactly the kept rows in slot order (V dim-major)
        Ki, Vi = p["K"][i], p["V"][i]
        rows = gidx[i]
        assert gK[i][:, :keep].tobytes() == np.ascontiguousarray(Ki[rows].transpose(1, 0, 2)).tobytes()
        assert gV[i][:, :, :keep].tobytes() == np.ascontiguousarray(Vi[rows].transpose(1, 2, 0)).tobytes()
        if n_diff:
            continue   # an in-band swap changes the evicted set; M is checked on the other sequences
        if i in (0, 3, 7):
            _, sm_ref = im.topk_select(Iref.astype(np.float32).astype(np.float64), cfg.B, cfg.R, cfg.recent_inclusive)
            ev = im.evicted_in_order(sm_ref)
            for gq in (0, 5) if i != 3 else (2,):
                refM, refb = im.memory_build(f(Ki[ev, gq]), f(Vi[ev, gq]), lam)
                assert normwise(gM[i, gq], refM) < 1e-4, f"seq {i} head {gq}: M"
                assert normwise(gb[i, gq], refb) < 1e-5, f"seq {i} head {gq}: b"


@pytest.mark.timeout(900)
def test_cfg3_decode_full_size(cfg3_layer):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, assert_output
    cfg, p = cfg3_layer
    f = lambda x: gen.from_storage(x, cfg.dtype)
    lam = float(np.float32(cfg.lam))
    keep = api.kvm_topk_keep(cfg.L, cfg.B, cfg.R, cfg.recent_inclusive)
    cap = api.cache_cap(keep + BENCH_T)
    dec = gen.make_decode(cfg, steps=DEC_STEPS)
    Kc = np.zeros((cfg.b, cfg.H_kv, cap, cfg.d))
    Vc = np.zeros((cfg.b, cfg.H_kv, cap, cfg.d))
    M = np.zeros((cfg.b, cfg.H_kv, cfg.d, cfg.d))
    bv = np.zeros((cfg.b, cfg.H_kv, cfg.d))
    pres = []
    for i in range(cfg.b):
        pre = im.prefill(f(p["X"][i]), f(p["Qwin"][i]), f(p["K"][i]), f(p["V"][i]), f(p["W_kI"]), p["gamma_k"],
                         f(p["W_qI"]), p["gamma_q"], f(p["W_g"]), cfg.B, cfg.R, lam, cfg.recent_inclusive,
                         eps=cfg.eps_rms, cap=cap)
        Kc[i], Vc[i], M[i], bv[i] = pre["Kc"], pre["Vc"], pre["M"], pre["b"]
        pres.append(pre)
    dK = to_dev(gen.to_storage(Kc, cfg.dtype))
    dV = to_dev(gen.to_storage(np.ascontiguousarray(Vc.transpose(0, 1, 3, 2)), cfg.dtype))
    dM, db = to_dev(M.astype(np.float32)), to_dev(bv.astype(np.float32))
    lens = to_dev(np.full(cfg.b, keep, np.int32))
    wg = to_dev(p["w_g"])
    outs = []
    for t in range(DEC_STEPS):
        o = api.kvm_decode_attn_mem(to_dev(dec["q"][t]), dK, dV, lens, k_new=to_dev(dec["k_new"][t]),
                                    v_new=to_dev(dec["v_new"][t]), M=dM, bvec=db, w_g=wg)
        api.kvm_len_add(lens, 1)
        outs.append(to_np(o))
    torch.cuda.synchronize()
    for i in range(cfg.b):
        M32, b32 = M[i].astype(np.float32).astype(np.float64), bv[i].astype(np.float32).astype(np.float64)
        ref, _, _, _ = im.decode(f(dec["q"][:, i]), f(dec["k_new"][:, i]), f(dec["v_new"][:, i]), pres[i]["Kc"],
                                 pres[i]["Vc"], keep, M32, b32, f(p["w_g"]))
        got = np.stack([o[i] for o in outs])
        assert_output(got, ref, cfg.dtype, f"seq {i}: o")
        np.testing.assert_allclose(got, ref, rtol=2e-4, atol=2e-4 * np.abs(ref).max())


CHUNK = 4096        # the benchmark's chunk for the chunked pre-eviction
CHUNK_SEQS = (0, 2, 5, 7)  # sequences checked against the oracle


@pytest.mark.timeout(900)
def test_cfg3_chunked_prefill_full_size(cfg3_layer):
    """Chunked pre-eviction of the full batch-8, 16384-token layer in chunks of 4096 tokens,
    in the benchmark's launch configuration (pool + chunk buffers of exactly keep + chunk
    rows, final caches of keep + 512 slots): for sampled sequences the kept set after every
    chunk, then the final caches (bit-exact), positions, importances, indexer keys and the
    memory of sampled KV heads, against the oracle's chunked prefill.  Each chunk's window
    queries are drawn N(0, 1) like the one-shot window's."""
    import torch
    from oracle import chunked as ck
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, set_check, normwise
    cfg, p = cfg3_layer
    f = lambda x: gen.from_storage(x, cfg.dtype)
    lam = float(np.float32(cfg.lam))
    L, W, B, R = cfg.L, cfg.W, cfg.B, cfg.R
    starts = list(range(0, L, CHUNK))
    r = gen.rng(211, cfg.cfg_id, L, CHUNK)
    Qw = [gen.to_storage(r.standard_normal((cfg.b, W, cfg.H_q, cfg.d)), cfg.dtype) for _ in starts]
    keep = api.kvm_topk_keep(L, B, R, cfg.recent_inclusive)
    cap = api.cache_cap(keep + BENCH_T)
    X, K, V = to_dev(p["X"]), to_dev(p["K"]), to_dev(p["V"])
    wts = [to_dev(p[k]) for k in ("W_kI", "gamma_k", "W_qI", "gamma_q", "W_g")]
    M = torch.zeros((cfg.b, cfg.H_kv, cfg.d, cfg.d), device="cuda")
    bv = torch.zeros((cfg.b, cfg.H_kv, cfg.d), device="cuda")
    P, pool, kept = 0, None, []
    for c, s0 in enumerate(starts):
        e = min(L, s0 + CHUNK)
        n = e - s0
        if pool is None:
            pool = dict(K=torch.empty((cfg.b, cfg.H_kv, n, cfg.d), dtype=torch.bfloat16, device="cuda"),
                        V=torch.empty((cfg.b, cfg.H_kv, n, cfg.d), dtype=torch.bfloat16, device="cuda"),
                        khat=torch.empty((cfg.b, n, cfg.d_I), device="cuda"),
                        I=torch.empty((cfg.b, n), device="cuda"),
                        pos=torch.empty((cfg.b, n), dtype=torch.int32, device="cuda"))
        last = c == len(starts) - 1
        cap_out = cap if last else min(P + n, B) + (min(L, starts[c + 1] + CHUNK) - starts[c + 1])
        pool, P = api.kvm_index_evict_chunk(X[:, s0:e].contiguous(), to_dev(Qw[c]), K[:, s0:e].contiguous(),
                                            V[:, s0:e].contiguous(), *wts, pool, P, s0, B, R, lam, cap_out, last,
                                            M, bv, recent_inclusive=cfg.recent_inclusive, eps=cfg.eps_rms)
        torch.cuda.synchronize()
        kept.append(to_np(pool["pos"])[:, :P].copy())
    assert P == keep
    gK, gV, gI, gkh, gM, gb = (to_np(t) for t in (pool["K"], pool["V"], pool["I"], pool["khat"], M, bv))
    Wk, Wq, Wg = f(p["W_kI"]), f(p["W_qI"]), f(p["W_g"])
    n_checked = 0
    for i in CHUNK_SEQS:
        Q = np.zeros((L, cfg.H_q, cfg.d), np.float32)   # the oracle reads only the windows
        for c, s0 in enumerate(starts):
            e = min(L, s0 + CHUNK)
            Q[e - W:e] = f(Qw[c][i])
        ref = ck.prefill_chunked(f(p["X"][i]), Q, f(p["K"][i]), f(p["V"][i]), Wk, p["gamma_k"], Wq, p["gamma_q"],
                                 Wg, B, R, lam, CHUNK, W, recent_inclusive=cfg.recent_inclusive, eps=cfg.eps_rms)
        del Q
        tie = False
        for c, st in enumerate(ref["steps"]):
            vidx = {int(t): j for j, t in enumerate(st["vpos"])}
            assert all(int(t) in vidx for t in kept[c][i]), f"seq {i} chunk {c}: position outside pool and chunk"
            if set_check([vidx[int(t)] for t in kept[c][i]], st["I"], B, R, cfg.recent_inclusive):
                tie = True   # an in-band swap changes every later chunk
                break
            np.testing.assert_array_equal(kept[c][i], st["kept"])
        if tie:
            continue
        n_checked += 1
        rows = ref["pos"]
        assert gK[i][:, :keep].tobytes() == np.ascontiguousarray(p["K"][i][rows].transpose(1, 0, 2)).tobytes()
        assert gV[i][:, :, :keep].tobytes() == np.ascontiguousarray(p["V"][i][rows].transpose(1, 2, 0)).tobytes()
        assert normwise(gI[i, :keep], ref["I"]) < 1e-5
        assert normwise(gkh[i, :keep], ref["k_hat"]) < 1e-5
        for g in (0, 3, 7):
            assert normwise(gM[i, g], ref["M"][g]) < 1e-4, f"seq {i} head {g}: M"
            assert normwise(gb[i, g], ref["b"][g]) < 1e-5, f"seq {i} head {g}: b"
    assert n_checked >= 1, "every sampled sequence met a near-tie"


@pytest.mark.timeout(900)
def test_stream_step_full_pool():
    """Streaming steps at the full pool (1024 + 64 slots) and model width of the 131072-token
    workload, from a synthetic pool state (positions spread over the prefix)."""
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise
    cfg = WORKLOADS["llama8b_layer_131k_stream"]
    dt = cfg.dtype
    lam = float(np.float32(cfg.lam))
    P = cfg.B + cfg.R
    cap = api.cache_cap(P)
    r = gen.rng(99, 0, 0, 0)
    w = gen.make_weights(cfg)
    f = lambda x: gen.from_storage(x, dt)
    older = np.sort(r.choice(cfg.L - cfg.R, size=cfg.B, replace=False))
    pos = np.concatenate([older, np.arange(cfg.L - cfg.R, cfg.L)]).astype(np.int64)
    kh = r.standard_normal((P, cfg.d_I))
    kh /= np.sqrt(np.mean(kh * kh, axis=1, keepdims=True))
    I0 = np.abs(r.standard_normal(P)) * 3
    Kc = f(gen.to_storage(r.standard_normal((cfg.H_kv, P, cfg.d)), dt))
    Vc = f(gen.to_storage(r.standard_normal((cfg.H_kv, P, cfg.d)), dt))
    M0 = r.standard_normal((cfg.H_kv, cfg.d, cfg.d)).astype(np.float32).astype(np.float64)
    b0 = np.abs(r.standard_normal((cfg.H_kv, cfg.d))).astype(np.float32).astype(np.float64)
    kh = kh.astype(np.float32).astype(np.float64)
    I0 = I0.astype(np.float32).astype(np.float64)
    st = so.StreamState(pos, I0, kh, Kc, Vc, M0, b0, cfg.L, cfg.R)
    Kd = np.zeros((1, cfg.H_kv, cap, cfg.d)); Kd[0, :, :P] = Kc
    Vd = np.zeros((1, cfg.H_kv, cap, cfg.d)); Vd[0, :, :P] = Vc
    dK = to_dev(gen.to_storage(Kd, dt))
    dV = to_dev(gen.to_storage(np.ascontiguousarray(Vd.transpose(0, 1, 3, 2)), dt))
    dM, db = to_dev(M0[None].astype(np.float32)), to_dev(b0[None].astype(np.float32))
    dkh, dI = to_dev(kh[None].astype(np.float32)), to_dev(I0[None].astype(np.float32))
    dpos, dnext = to_dev(pos[None].astype(np.int32)), to_dev(np.array([cfg.L], np.int32))
    lens = to_dev(np.array([P], np.int32))
    wts = [to_dev(w[k]) for k in ("W_kI", "gamma_k", "W_qI", "gamma_q", "W_g")]
    dec = gen.make_decode(cfg, steps=6)
    for t in range(6):
        x_t, q_t, k_t, v_t = dec["x_new"][t], dec["q"][t], dec["k_new"][t], dec["v_new"][t]
        e = api.kvm_stream_evict(to_dev(x_t), to_dev(q_t), *wts, dkh, dI, dpos, dnext, dK, dV, dM, db, lam, cfg.R,
                                 eps=cfg.eps_rms)
        o = api.kvm_decode_attn_mem(to_dev(q_t), dK, dV, lens, k_new=to_dev(k_t), v_new=to_dev(v_t),
                                    append_slot=e, M=dM, bvec=db, w_g=to_dev(w["w_g"]))
        torch.cuda.synchronize()
        o_ref, _, _, e_ref = so.step(st, f(x_t[0]), f(q_t[0]), f(k_t[0]), f(v_t[0]), f(w["W_kI"]), w["gamma_k"],
                                     f(w["W_qI"]), w["gamma_q"], f(w["W_g"]), f(w["w_g"]), lam, cfg.eps_rms)
        assert int(to_np(e)[0]) == e_ref, f"step {t}: evicted slot"
        np.testing.assert_array_equal(to_np(dpos)[0], st.slot_pos)
        assert normwise(to_np(dI)[0], st.I) < 1e-5
        assert normwise(to_np(dM)[0], st.M) < 1e-5
        np.testing.assert_allclose(to_np(o)[0], o_ref, rtol=2e-4, atol=2e-4 * np.abs(o_ref).max())


@pytest.mark.timeout(900)
def test_momentkv_alpha_full_size():
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise
    cfg = WORKLOADS["qwen3_4b_momentkv_32k"].with_(layers=1)
    p = gen.make_prefill(cfg)
    al = to_np(api.kvm_moment_alpha(to_dev(p["Qwin"]), to_dev(p["K"])))
    torch.cuda.synchronize()
    f = lambda x: gen.from_storage(x, cfg.dtype)
    np.testing.assert_allclose(al.sum(-1), 1.0, rtol=1e-4)
    G = cfg.H_q // cfg.H_kv
    for i, g in ((0, 0), (3, 7)):
        Q = f(p["Qwin"][i][:, g * G:(g + 1) * G])
        K = f(p["K"][i][:, g:g + 1])
        ref = mk.alpha(Q, K, np.arange(cfg.L - cfg.W, cfg.L), 1 / math.sqrt(cfg.d), G)[0]
        assert normwise(al[i, g], ref) < 1e-5, f"alpha ({i}, {g})"
        np.testing.assert_allclose(al[i, g], ref, rtol=1e-4, atol=1e-6 * ref.max())
