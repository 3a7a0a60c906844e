"""Checkpoint and resume of the decode-time state.  The library keeps no state of its own:
everything a decode step needs (caches, latent memory or moment sums, the pool's indexer
keys, importances and positions, lengths) is caller-owned device memory.  A checkpoint is
therefore those tensors written to a file; resuming loads them into fresh device buffers.
Each test runs T steps without interruption, then again from the same start with a
checkpoint written to disk, every device buffer dropped and reloaded half way, and
requires bitwise-identical outputs, evictions and final state (the kernels use no atomics,
so repeated runs are bitwise reproducible)."""
import numpy as np
import pytest

from synth import WORKLOADS, gen

pytestmark = pytest.mark.gpu


def _save(path, state):
    """Device tensors -> .npz (bf16 as its bit pattern)."""
    import torch
    arrays, kinds = {}, {}
    for k, t in state.items():
        if t.dtype == torch.bfloat16:
            arrays[k] = t.view(torch.int16).cpu().numpy()
            kinds[k] = "bf16"
        else:
            arrays[k] = t.cpu().numpy()
    np.savez(path, **arrays)
    return kinds


def _load(path, kinds):
    import torch
    out = {}
    with np.load(path) as z:     # allow_pickle stays False
        for k in z.files:
            t = torch.from_numpy(np.ascontiguousarray(z[k])).cuda()
            out[k] = t.view(torch.bfloat16) if kinds.get(k) == "bf16" else t
    return out


def _clone(state):
    return {k: v.clone() for k, v in state.items()}


def _run_stream(api, st, steps, inputs, wts, lam, R, w_g):
    import torch
    outs, evs = [], []
    for (x, q, k, v) in steps:
        e = api.kvm_stream_evict(x, q, *wts, st["khat"], st["I"], st["pos"], st["npos"], st["Kc"], st["Vc"], st["M"],
                                 st["b"], lam, R)
        o = api.kvm_decode_attn_mem(q, st["Kc"], st["Vc"], st["lens"], k_new=k, v_new=v, append_slot=e, M=st["M"],
                                    bvec=st["b"], w_g=w_g)
        outs.append(o.clone())
        evs.append(e.clone())
    torch.cuda.synchronize()
    return outs, evs


def test_streaming_checkpoint_resume(tmp_path):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev
    cfg = WORKLOADS["llama8b_layer_131k_stream"].with_(L=4096)
    lam = float(np.float32(cfg.lam))
    T, T1 = 24, 10
    p = gen.make_prefill(cfg)
    dec = gen.make_decode(cfg, steps=T)
    wts = [to_dev(p[k]) for k in ("W_kI", "gamma_k", "W_qI", "gamma_q", "W_g")]
    w_g = to_dev(p["w_g"])
    khat = torch.empty((1, cfg.L, cfg.d_I), device="cuda")
    I = api.kvm_index_score(to_dev(p["X"]), to_dev(p["Qwin"]), *wts, khat=khat, eps=cfg.eps_rms)
    idx, sm = api.kvm_topk_select(I, cfg.B, cfg.R, cfg.recent_inclusive)
    P = idx.shape[1]
    M = torch.zeros((1, cfg.H_kv, cfg.d, cfg.d), device="cuda")
    bv = torch.zeros((1, cfg.H_kv, cfg.d), device="cuda")
    Kc, Vc = api.kvm_compact_kv(to_dev(p["K"]), to_dev(p["V"]), sm, idx, P, api.cache_cap(P), M=M, bvec=bv, lam=lam)
    start = dict(Kc=Kc, Vc=Vc, M=M, b=bv, khat=api.kvm_gather_rows(khat, sm, P), I=api.kvm_gather_rows(I, sm, P),
                 pos=api.kvm_gather_rows(torch.arange(cfg.L, dtype=torch.int32, device="cuda")[None].contiguous(),
                                         sm, P),
                 npos=to_dev(np.array([cfg.L], np.int32)), lens=to_dev(np.array([P], np.int32)))
    steps = [(to_dev(dec["x_new"][t]), to_dev(dec["q"][t]), to_dev(dec["k_new"][t]), to_dev(dec["v_new"][t]))
             for t in range(T)]
    # uninterrupted
    a = _clone(start)
    outs_a, evs_a = _run_stream(api, a, steps, None, wts, lam, cfg.R, w_g)
    # checkpoint after T1 steps, drop every device buffer, reload, continue
    bst = _clone(start)
    outs_b, evs_b = _run_stream(api, bst, steps[:T1], None, wts, lam, cfg.R, w_g)
    kinds = _save(tmp_path / "stream.npz", bst)
    del bst
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    bst = _load(tmp_path / "stream.npz", kinds)
    o2, e2 = _run_stream(api, bst, steps[T1:], None, wts, lam, cfg.R, w_g)
    outs_b += o2
    evs_b += e2
    for t in range(T):
        assert torch.equal(evs_a[t], evs_b[t]), f"step {t}: evicted slot"
        assert outs_a[t].view(torch.int32).equal(outs_b[t].view(torch.int32)), f"step {t}: output bits"
    for k in start:
        x, y = a[k], bst[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        elif x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), f"final state {k}"


def test_momentkv_stream_checkpoint_resume(tmp_path):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev
    b, H_q, H_kv, d, P, R, T, T1 = 2, 32, 8, 128, 256, 16, 20, 7
    r = gen.rng(192, 0, 0, 0)
    st = lambda x: to_dev(gen.to_storage(x, "bf16"))
    cap = api.cache_cap(P)
    Kc = np.zeros((b, H_kv, cap, d)); Kc[:, :, :P] = r.standard_normal((b, H_kv, P, d))
    Vc = np.zeros((b, H_kv, cap, d)); Vc[:, :, :P] = r.standard_normal((b, H_kv, P, d))
    L0 = 4 * P
    pos = np.stack([np.stack([np.sort(r.choice(L0, P, replace=False)) for _ in range(H_kv)]) for _ in range(b)])
    n0 = 40
    Ke, Ve = r.standard_normal((b, H_kv, n0, d)), r.standard_normal((b, H_kv, n0, d))
    start = dict(Kc=st(Kc), Vc=st(np.ascontiguousarray(Vc.transpose(0, 1, 3, 2))),
                 pos=to_dev(pos.astype(np.int32)), npos=to_dev(np.full(b, L0, np.int32)),
                 n_e=to_dev(np.full((b, H_kv), n0, np.int32)), s_k=to_dev(Ke.sum(2).astype(np.float32)),
                 s_v=to_dev(Ve.sum(2).astype(np.float32)),
                 S=to_dev(np.einsum("bgnv,bgnk->bgvk", Ve, Ke).astype(np.float32)),
                 lens=to_dev(np.full(b, P, np.int32)))
    steps = [(st(r.standard_normal((b, H_q, d))), st(r.standard_normal((b, H_kv, d))),
              st(r.standard_normal((b, H_kv, d)))) for _ in range(T)]

    def run(s, part):
        outs, evs = [], []
        for (q, k, v) in part:
            mom = dict(n_e=s["n_e"], s_k=s["s_k"], s_v=s["s_v"], S=s["S"])
            e = api.kvm_moment_stream_evict(q, k, v, s["Kc"], s["Vc"], s["pos"], s["npos"], mom, R)
            o = api.kvm_decode_attn_mem(q, s["Kc"], s["Vc"], s["lens"], moments=mom)
            outs.append(o.clone())
            evs.append(e.clone())
        torch.cuda.synchronize()
        return outs, evs

    a = _clone(start)
    outs_a, evs_a = run(a, steps)
    bst = _clone(start)
    outs_b, evs_b = run(bst, steps[:T1])
    kinds = _save(tmp_path / "mstream.npz", bst)
    del bst
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    bst = _load(tmp_path / "mstream.npz", kinds)
    o2, e2 = run(bst, steps[T1:])
    outs_b += o2
    evs_b += e2
    for t in range(T):
        assert torch.equal(evs_a[t], evs_b[t]), f"step {t}: evicted slots"
        assert outs_a[t].view(torch.int32).equal(outs_b[t].view(torch.int32)), f"step {t}: output bits"
    for k in start:
        x, y = a[k], bst[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        elif x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), f"final state {k}"
