"""GPU pipelines shared by the parity tests: the calls a caller makes, in order, with the
intermediate results copied back for comparison.  Nothing here computes any part of the
method; every step is a libkvmem entry point."""
import math

import numpy as np

from oracle import momentkv as mk
from synth import gen


def momentkv_prefill_gpu(Q, Kt, Vt, B, cap):
    """Moment-informed prefill on the GPU: alpha once, then halving rounds of residual
    score -> per-head top-k -> compaction with the moment fold, until B tokens remain.
    Q [b,W,H_q,d], Kt, Vt [b,L,H_kv,d] device bf16.  Returns alpha (numpy), the rounds as
    (scores [b*H_kv, n], kept local indices [b*H_kv, keep]) numpy pairs, the kept
    positions [b*H_kv, B], the moments (device dict) and the final caches (Kc, Vc)."""
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_np
    b, L, H, d = Kt.shape
    alpha = api.kvm_moment_alpha(Q, Kt)
    mom = dict(n_e=torch.zeros((b, H), dtype=torch.int32, device=Kt.device),
               s_k=torch.zeros((b, H, d), device=Kt.device), s_v=torch.zeros((b, H, d), device=Kt.device),
               S=torch.zeros((b, H, d, d), device=Kt.device))
    Kc, Vc = Kt, Vt
    al = alpha.view(b * H, L)
    pos = torch.arange(L, dtype=torch.int32, device=Kt.device).repeat(b * H, 1).contiguous()
    n, hm = L, False
    rounds = []
    while n > B:
        keep = max(B, -(-n // 2))
        last = keep == B
        sc = api.kvm_moment_score(Kc, Vc, al.view(b, H, n), mom, kv_head_major=hm)
        idx, sm = api.kvm_topk_select(sc.view(b * H, n), keep, 0)
        rounds.append((to_np(sc).reshape(b * H, n), to_np(idx)))
        Kn, Vn = api.kvm_compact_kv(Kc, Vc, sm, idx, keep, cap=cap if last else keep, moments=mom, per_head=True,
                                    kv_head_major=hm, v_row_major=not last)
        al = api.kvm_gather_rows(al, sm, keep)
        pos = api.kvm_gather_rows(pos, sm, keep)
        Kc, Vc, n, hm = Kn, Vn, keep, True
    torch.cuda.synchronize()
    return to_np(alpha), rounds, to_np(pos), mom, Kc, Vc


def kept_check(gpu_kept, scores_ref, keep, rel=1e-5):
    """Per-head round decision: the GPU's kept set equals the oracle's top `keep` of its
    scores rounded to fp32 (the kernel's precision) outside the band within `rel` of the
    keep-th score.  Returns the number of in-band differences."""
    s32 = np.asarray(scores_ref, np.float64).astype(np.float32).astype(np.float64)
    ref_kept, _ = mk.select_round(s32, np.arange(len(s32)), keep)
    g, rf = set(int(x) for x in gpu_kept), set(int(x) for x in ref_kept)
    assert len(g) == len(rf)
    tau = min(s32[j] for j in ref_kept)
    band = np.abs(s32 - tau) <= rel * abs(tau)
    bad = [j for j in g ^ rf if not band[j]]
    assert not bad, f"kept-set mismatch outside the band at {bad[:8]}"
    return len(g ^ rf)


def momentkv_compare(p, pairs, B, T, dec, cap):
    """The moment-informed prefill and T decode steps with the NC mix on the GPU, against
    the oracle run per sampled (sequence, KV head) pair.  A pair is compared round by round
    (scores, kept set) until an in-band difference (a near-tie the 1e-5 rule allows): from
    there the two states legitimately differ and that pair is no longer compared.  Pairs
    that stay identical through every round are then checked for their kept positions,
    moments and every decode output of their query heads.  Returns (pairs compared through
    decode, total rounds compared)."""
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise, assert_output
    f = lambda x: gen.from_storage(x, "bf16")
    Q, Kt, Vt = p["Qwin"], p["K"], p["V"]
    b, L, H, d = Kt.shape
    G = Q.shape[2] // H
    alpha, rounds, g_pos, mom, Kc, Vc = momentkv_prefill_gpu(to_dev(Q), to_dev(Kt), to_dev(Vt), B, cap)
    g_mom = {k: to_np(v) for k, v in mom.items()}
    refs = {}
    live = {}
    n_rounds = 0
    for (i, g) in pairs:
        ref = mk.prefill(f(Q[i][:, g * G:(g + 1) * G]), f(Kt[i][:, g:g + 1]), f(Vt[i][:, g:g + 1]), B)
        refs[(i, g)] = ref
        assert normwise(alpha[i, g], ref["alpha"][0]) < 1e-5, f"alpha ({i}, {g})"
        hd = ref["heads"][0]
        assert len(hd["rounds"]) == len(rounds) == mk.n_rounds(L, B)
        live[(i, g)] = True
        for r, (g_sc, g_idx) in enumerate(rounds):
            rr = hd["rounds"][r]
            row = i * H + g
            assert normwise(g_sc[row], rr["scores"]) < 1e-5, f"round {r} scores ({i}, {g})"
            n_rounds += 1
            if kept_check(g_idx[row], rr["scores"], len(rr["kept"])):
                live[(i, g)] = False
                break
        if not live[(i, g)]:
            continue
        np.testing.assert_array_equal(np.sort(g_pos[i * H + g][:B]), hd["kept"])
        m = hd["mom"]
        assert int(g_mom["n_e"][i, g]) == m["n"]
        assert normwise(g_mom["S"][i, g], m["S"]) < 1e-5, f"S ({i}, {g})"
        assert normwise(g_mom["s_k"][i, g], m["sk"]) < 1e-5, f"s_k ({i}, {g})"
        assert normwise(g_mom["s_v"][i, g], m["sv"]) < 1e-5, f"s_v ({i}, {g})"
    # decode with the NC mix over each head's retained tokens (all heads run on the GPU)
    lens = torch.full((b,), B, dtype=torch.int32, device=Kc.device)
    outs = []
    for t in range(T):
        o = api.kvm_decode_attn_mem(to_dev(dec["q"][t]), Kc, Vc, lens, k_new=to_dev(dec["k_new"][t]),
                                    v_new=to_dev(dec["v_new"][t]), moments=mom)
        outs.append(to_np(o))
        api.kvm_len_add(lens, 1)
    torch.cuda.synchronize()
    n_dec = 0
    for (i, g), ok in live.items():
        if not ok:
            continue
        hs = slice(g * G, (g + 1) * G)
        ref, _, _ = mk.decode(f(dec["q"][:, i, hs]), f(dec["k_new"][:, i, g:g + 1]), f(dec["v_new"][:, i, g:g + 1]),
                              f(Kt[i][:, g:g + 1]), f(Vt[i][:, g:g + 1]), refs[(i, g)]["heads"])
        got = np.stack([o[i, hs] for o in outs])
        assert_output(got, ref, "bf16", f"MomentKV decode ({i}, {g})")
        np.testing.assert_allclose(got, ref, rtol=1e-3, atol=1e-3 * np.abs(ref).max())
        n_dec += 1
    return n_dec, n_rounds
