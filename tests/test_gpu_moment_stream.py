"""kvm_moment_stream_evict + kvm_decode_attn_mem (moments mode) against the oracle's
MomentKV decode step, step by step, per (sequence, KV head).

Both sides start from the same pool (bf16 K/V, positions) and the same fp32 moments.
Decision rule: the evicted slot must equal the oracle's, decided on the oracle's scores
rounded to fp32 (the kernel's precision), unless the two slots' scores lie within 1e-5 of
each other; after such a near-tie the pair's states legitimately diverge, so that pair's
comparison stops there, after at least 8 compared steps."""
import numpy as np
import pytest

from oracle import moment_stream as ms
from oracle import momentkv as mk
from synth import WORKLOADS, gen

pytestmark = pytest.mark.gpu

BF = "bf16"


def _f32_moms(moms):
    return [dict(n=m["n"], sk=np.float32(m["sk"]).astype(np.float64), sv=np.float32(m["sv"]).astype(np.float64),
                 S=np.float32(m["S"]).astype(np.float64)) for m in moms]


def _synthetic_pool(b, H_kv, d, P, n_ev, seed):
    """Per sequence: positions (distinct, below 4P), bf16 K/V rows and the moments of n_ev
    evicted bf16 rows per KV head."""
    r = gen.rng(190, seed, 0, 0)
    L0 = 4 * P
    out = []
    for _ in range(b):
        pos = np.stack([np.sort(r.choice(L0, P, replace=False)) for _ in range(H_kv)])
        Kc = gen.from_storage(gen.to_storage(r.standard_normal((H_kv, P, d)), BF), BF)
        Vc = gen.from_storage(gen.to_storage(r.standard_normal((H_kv, P, d)), BF), BF)
        moms = []
        for _ in range(H_kv):
            m = mk.empty(d)
            if n_ev:
                m = mk.add(m, gen.from_storage(gen.to_storage(r.standard_normal((n_ev, d)), BF), BF),
                           gen.from_storage(gen.to_storage(r.standard_normal((n_ev, d)), BF), BF))
            moms.append(m)
        out.append((pos, Kc, Vc, _f32_moms(moms), L0))
    return out


def _prefill_pool(cfg):
    """Pools from the oracle's moment-informed prefill of the MomentKV workload's inputs."""
    p = gen.make_prefill(cfg)
    f = lambda x: gen.from_storage(x, BF)
    out = []
    for i in range(cfg.b):
        pre = mk.prefill(f(p["Qwin"][i]), f(p["K"][i]), f(p["V"][i]), cfg.B)
        st = ms.from_prefill(pre, f(p["K"][i]), f(p["V"][i]), cfg.L, 0)
        out.append((st.slot_pos, st.Kc, st.Vc, _f32_moms(st.moms), cfg.L))
    return out


def _steps(b, H_q, H_kv, d, T, seed):
    r = gen.rng(191, seed, 0, 0)
    st = lambda *s: gen.to_storage(r.standard_normal(s), BF)
    return st(T, b, H_q, d), st(T, b, H_kv, d), st(T, b, H_kv, d)


CASES = [
    # name, b, H_q, H_kv, d, P (None: from the prefill), R, steps, initial evictions
    ("prefill_qwen_shape", 2, 32, 8, 128, None, 0, 24, 0),
    ("pool1024_window16", 1, 32, 8, 128, 1024, 16, 12, 3000),
    ("d64_ragged_empty_moments", 2, 8, 2, 64, 200, 5, 16, 0),
    ("G1", 1, 8, 8, 128, 300, 0, 12, 50),
    ("G8_ragged_by_one", 1, 16, 2, 64, 129, 0, 16, 20),
    # grids of >= 256 blocks of 128 slots: the score kernel's wide-block variant
    ("pool1024_batch4_wide_blocks", 4, 32, 8, 128, 1024, 16, 5, 2000),
    ("d64_wide_blocks_ragged", 4, 8, 8, 64, 1000, 0, 4, 300),
]


@pytest.mark.parametrize("name,b,H_q,H_kv,d,P,R,T,n_ev", CASES, ids=[c[0] for c in CASES])
def test_moment_stream_steps_match_oracle(name, b, H_q, H_kv, d, P, R, T, n_ev):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise, assert_output

    if P is None:
        cfg = WORKLOADS["qwen3_4b_momentkv_32k"].with_(L=1024, B=128, b=b, T=T)
        pools = _prefill_pool(cfg)
        qs, ks, vs = (gen.make_decode(cfg, steps=T)[k] for k in ("q", "k_new", "v_new"))
    else:
        pools = _synthetic_pool(b, H_kv, d, P, n_ev, seed=P + d)
        qs, ks, vs = _steps(b, H_q, H_kv, d, T, seed=P + T)
    P = pools[0][0].shape[1]
    cap = api.cache_cap(P)
    sts = [ms.MomentStreamState(pos, Kc, Vc, moms, L0, R) for pos, Kc, Vc, moms, L0 in pools]

    Kc = np.zeros((b, H_kv, cap, d))
    Vc = np.zeros((b, H_kv, d, cap))
    for i, st in enumerate(sts):
        Kc[i, :, :P] = st.Kc
        Vc[i, :, :, :P] = st.Vc.transpose(0, 2, 1)
    dKc, dVc = to_dev(gen.to_storage(Kc, BF)), to_dev(gen.to_storage(Vc, BF))
    dpos = to_dev(np.stack([st.slot_pos for st in sts]).astype(np.int32))
    dnext = to_dev(np.array([st.next_pos for st in sts], np.int32))
    mom = dict(n_e=to_dev(np.array([[m["n"] for m in st.moms] for st in sts], np.int32)),
               s_k=to_dev(np.array([[m["sk"] for m in st.moms] for st in sts], np.float32)),
               s_v=to_dev(np.array([[m["sv"] for m in st.moms] for st in sts], np.float32)),
               S=to_dev(np.array([[m["S"] for m in st.moms] for st in sts], np.float32)))
    lens = to_dev(np.full(b, P, np.int32))
    G = H_q // H_kv
    f = lambda x: gen.from_storage(x, BF)

    live = np.ones((b, H_kv), bool)
    compared = np.zeros((b, H_kv), int)
    for t in range(T):
        e_dev = api.kvm_moment_stream_evict(to_dev(qs[t]), to_dev(ks[t]), to_dev(vs[t]), dKc, dVc, dpos, dnext,
                                            mom, R)
        o = api.kvm_decode_attn_mem(to_dev(qs[t]), dKc, dVc, lens, moments=mom)
        torch.cuda.synchronize()
        g_e, g_pos, g_o = to_np(e_dev), to_np(dpos), to_np(o)
        g_K, g_V = f(to_np(dKc)), f(to_np(dVc))
        g_n, g_sk, g_sv, g_S = (to_np(mom[k]) for k in ("n_e", "s_k", "s_v", "S"))
        assert np.array_equal(to_np(dnext), [st.next_pos + 1 for st in sts])
        for i, st in enumerate(sts):
            p = st.next_pos
            pos_before = st.slot_pos.copy()
            o_ref, _, e_ref, _, scores = ms.step(st, f(qs[t][i]), f(ks[t][i]), f(vs[t][i]))
            for g in range(H_kv):
                if not live[i, g]:
                    continue
                eg, er = int(g_e[i, g]), int(e_ref[g])
                if eg != er:
                    s32 = scores[g].astype(np.float32).astype(np.float64)
                    assert pos_before[g, eg] <= p - R, f"step {t} ({i},{g}): slot {eg} is in the recent window"
                    assert abs(s32[eg] - s32[er]) <= 1e-5 * abs(s32[er]), \
                        f"step {t} ({i},{g}): evicted {eg} (score {s32[eg]}) != oracle {er} (score {s32[er]})"
                    assert compared[i, g] >= min(8, T), f"({i},{g}) near-tie after {compared[i, g]} steps"
                    live[i, g] = False
                    continue
                np.testing.assert_array_equal(g_pos[i, g], st.slot_pos[g])
                np.testing.assert_array_equal(g_K[i, g, :P], st.Kc[g])
                np.testing.assert_array_equal(g_V[i, g, :, :P], st.Vc[g].T)
                m = st.moms[g]
                assert g_n[i, g] == m["n"]
                assert normwise(g_sk[i, g], m["sk"]) < 1e-5 and normwise(g_sv[i, g], m["sv"]) < 1e-5
                assert normwise(g_S[i, g], m["S"]) < 1e-5, f"step {t} ({i},{g}): S"
                for h in range(g * G, (g + 1) * G):
                    assert_output(g_o[i, h], o_ref[h], BF, f"step {t} ({i},{h}): o")
                    np.testing.assert_allclose(g_o[i, h], o_ref[h], rtol=2e-4, atol=2e-4 * np.abs(o_ref[h]).max())
                compared[i, g] += 1
    assert compared.min() >= min(8, T)
