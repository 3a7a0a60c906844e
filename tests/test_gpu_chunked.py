"""Chunked pre-eviction (kvm_index_evict_chunk) against the oracle's chunked prefill, chunk by
chunk: the kept set after every chunk (exact outside the 1e-5 band of the selection
threshold, decided on the oracle's importances rounded to fp32), then the final pool's
caches (bit-exact), positions, importances, indexer keys and the latent memory.

A difference inside the band legitimately changes every later chunk, so a sequence's
comparison stops there (after at least one compared chunk).  Inputs: the workloads'
generators for X, K, V and the weights; model queries for every position drawn from the
same N(0, 1) distribution."""
import numpy as np
import pytest

from oracle import chunked as ck
from synth import WORKLOADS, gen

pytestmark = pytest.mark.gpu

CASES = [
    # workload, overrides, chunk, batch elements
    ("llama8b_layer_4k", dict(L=1500, B=300, R=32, needles=0), 512, 2),
    ("llama8b_layer_4k", dict(L=1200, B=256, R=32, needles=0), 1200, 1),   # one chunk: the one-shot pre-eviction
    ("tiny_fp32", dict(L=512, B=64, R=0), 128, 1),                  # fp32, the fused-multiply-add kernels
    ("tiny_fp32", dict(L=400, B=90, R=16), 100, 2),
]


@pytest.mark.parametrize("wl,over,C,nb", CASES)
def test_chunked_pre_eviction_matches_oracle(wl, over, C, nb):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise, set_check

    cfg = WORKLOADS[wl].with_(**over)
    dt, L, W, B, R = cfg.dtype, cfg.L, cfg.W, cfg.B, cfg.R
    lam = float(np.float32(cfg.lam))
    bl = list(range(nb))
    p = gen.make_prefill(cfg, batches=bl)
    r = gen.rng(210, cfg.cfg_id, L, C)
    Q = gen.to_storage(r.standard_normal((nb, L, cfg.H_q, cfg.d)), dt)
    f = lambda x: gen.from_storage(x, dt)
    W_kI, W_qI, W_g = f(p["W_kI"]), f(p["W_qI"]), f(p["W_g"])
    refs = [ck.prefill_chunked(f(p["X"][i]), f(Q[i]), f(p["K"][i]), f(p["V"][i]), W_kI, p["gamma_k"], W_qI,
                               p["gamma_q"], W_g, B, R, lam, C, W, eps=cfg.eps_rms) for i in bl]

    X, Qd, K, V = to_dev(p["X"]), to_dev(Q), to_dev(p["K"]), to_dev(p["V"])
    wts = [to_dev(p[k]) for k in ("W_kI", "gamma_k", "W_qI", "gamma_q", "W_g")]
    M = torch.zeros((nb, cfg.H_kv, cfg.d, cfg.d), device="cuda")
    bv = torch.zeros((nb, cfg.H_kv, cfg.d), device="cuda")
    starts = list(range(0, L, C))
    cap = api.cache_cap(min(B, L))
    P, pool = 0, None
    live = [True] * nb
    compared = [0] * nb
    for c, s0 in enumerate(starts):
        e = min(L, s0 + C)
        n = e - s0
        if pool is None:
            tdt = torch.bfloat16 if dt == "bf16" else torch.float32
            pool = dict(K=torch.empty((nb, cfg.H_kv, n, cfg.d), dtype=tdt, device="cuda"),
                        V=torch.empty((nb, cfg.H_kv, n, cfg.d), dtype=tdt, device="cuda"),
                        khat=torch.empty((nb, n, cfg.d_I), device="cuda"),
                        I=torch.empty((nb, n), device="cuda"),
                        pos=torch.empty((nb, n), dtype=torch.int32, device="cuda"))
        last = c == len(starts) - 1
        keep = min(P + n, B)
        cap_out = cap if last else keep + (min(L, starts[c + 1] + C) - starts[c + 1])
        pool, P = api.kvm_index_evict_chunk(X[:, s0:e].contiguous(), Qd[:, e - W:e].contiguous(),
                                            K[:, s0:e].contiguous(), V[:, s0:e].contiguous(), *wts, pool, P, s0,
                                            B, R, lam, cap_out, last, M, bv, eps=cfg.eps_rms)
        assert P == keep
        torch.cuda.synchronize()
        g_pos = to_np(pool["pos"])[:, :P]
        for i in bl:
            if not live[i]:
                continue
            st = refs[i]["steps"][c]
            vidx = {int(t): j for j, t in enumerate(st["vpos"])}
            assert all(int(t) in vidx for t in g_pos[i]), f"chunk {c}: pooled position outside pool and chunk"
            n_band = set_check([vidx[int(t)] for t in g_pos[i]], st["I"], B, R)
            if n_band:
                assert compared[i] >= 1, f"seq {i}: near-tie at the first chunk"
                live[i] = False
                continue
            np.testing.assert_array_equal(g_pos[i], st["kept"])
            compared[i] += 1
    assert any(live), "every sequence stopped at a near-tie"

    # (slots past the kept count hold whatever the pool's allocation held: not converted)
    gK, gV = to_np(pool["K"]), to_np(pool["V"])
    gI, gkh = to_np(pool["I"]), to_np(pool["khat"])
    gM, gb = to_np(M), to_np(bv)
    for i in bl:
        if not live[i]:
            continue
        ref = refs[i]
        n = len(ref["pos"])
        np.testing.assert_array_equal(f(gK[i, :, :n]), ref["K"].transpose(1, 0, 2))
        np.testing.assert_array_equal(f(gV[i, :, :, :n]), ref["V"].transpose(1, 2, 0))
        assert normwise(gI[i, :n], ref["I"]) < 1e-5
        assert normwise(gkh[i, :n], ref["k_hat"]) < 1e-5
        for g in range(cfg.H_kv):
            bar = 1e-4 if dt == "bf16" else 1e-5   # bf16: the hi + lo split of lam^(n-i) phi(k)
            assert normwise(gM[i, g], ref["M"][g]) < bar
            assert normwise(gb[i, g], ref["b"][g]) < bar


def test_chunked_in_place_matches_copy():
    """The chunk's K/V already in the pool's rows P .. P+C-1 (K = V = NULL) gives the same pools,
    caches and memory, bit for bit, as handing the chunk's token-major K/V to the call."""
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev

    cfg = WORKLOADS["llama8b_layer_4k"].with_(L=1500, B=300, R=32, needles=0)
    C, nb, W = 512, 2, cfg.W
    p = gen.make_prefill(cfg, batches=list(range(nb)))
    r = gen.rng(212, cfg.cfg_id, cfg.L, C)
    Qd = to_dev(gen.to_storage(r.standard_normal((nb, cfg.L, cfg.H_q, cfg.d)), cfg.dtype))
    X, K, V = to_dev(p["X"]), to_dev(p["K"]), to_dev(p["V"])
    wts = [to_dev(p[k]) for k in ("W_kI", "gamma_k", "W_qI", "gamma_q", "W_g")]
    cap = api.cache_cap(min(cfg.B, cfg.L))
    starts = list(range(0, cfg.L, C))
    outs = []
    for in_place in (False, True):
        M = torch.zeros((nb, cfg.H_kv, cfg.d, cfg.d), device="cuda")
        bv = torch.zeros((nb, cfg.H_kv, cfg.d), device="cuda")
        P, pool = 0, None
        for c, s0 in enumerate(starts):
            e = min(cfg.L, s0 + C)
            n = e - s0
            if pool is None:
                pool = dict(K=torch.empty((nb, cfg.H_kv, n, cfg.d), dtype=torch.bfloat16, device="cuda"),
                            V=torch.empty((nb, cfg.H_kv, n, cfg.d), dtype=torch.bfloat16, device="cuda"),
                            khat=torch.empty((nb, n, cfg.d_I), device="cuda"),
                            I=torch.empty((nb, n), device="cuda"),
                            pos=torch.empty((nb, n), dtype=torch.int32, device="cuda"))
            last = c == len(starts) - 1
            cap_out = cap if last else min(P + n, cfg.B) + (min(cfg.L, starts[c + 1] + C) - starts[c + 1])
            Kc, Vc = K[:, s0:e].contiguous(), V[:, s0:e].contiguous()
            if in_place:   # the chunk's rows written into the pool tail, head-major
                pool["K"][:, :, P:P + n] = Kc.transpose(1, 2)
                pool["V"][:, :, P:P + n] = Vc.transpose(1, 2)
                Kc = Vc = None
            pool, P = api.kvm_index_evict_chunk(X[:, s0:e].contiguous(), Qd[:, e - W:e].contiguous(), Kc, Vc, *wts,
                                                pool, P, s0, cfg.B, cfg.R, float(np.float32(cfg.lam)), cap_out, last,
                                                M, bv, eps=cfg.eps_rms)
        torch.cuda.synchronize()
        outs.append({**{k: v[..., :P] if k != "V" else v[..., :P] for k, v in pool.items() if k in ("I", "pos")},
                     "K": pool["K"][:, :, :P].clone(), "V": pool["V"][:, :, :, :P].clone(),
                     "khat": pool["khat"][:, :P].clone(), "M": M.clone(), "b": bv.clone()})
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k]), k
