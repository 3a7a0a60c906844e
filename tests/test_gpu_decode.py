"""kvm_decode_attn_mem against the oracle: split-K attention with (a, lse) merge and the
memory read-out, on seeded inputs of the workloads' shapes."""
import math

import numpy as np
import pytest

from oracle import indexmem as im
from synth import gen

pytestmark = pytest.mark.gpu


def _case(dtype, b, H_q, H_kv, d, cap, lens, seed, n_ev=50, lam=0.99):
    r = gen.rng(90, seed, 0, 0)
    st = lambda x: gen.to_storage(x, dtype)
    Kc = st(r.standard_normal((b, H_kv, cap, d)))
    Vc = st(r.standard_normal((b, H_kv, cap, d)))
    q = st(r.standard_normal((b, H_q, d)))
    kn = st(r.standard_normal((b, H_kv, d)))
    vn = st(r.standard_normal((b, H_kv, d)))
    w_g = st(r.standard_normal((H_q, d)) / math.sqrt(d))
    M = np.zeros((b, H_kv, d, d))
    bv = np.zeros((b, H_kv, d))
    for bi in range(b):
        for g in range(H_kv):
            M[bi, g], bv[bi, g] = im.memory_build(r.standard_normal((n_ev, d)), r.standard_normal((n_ev, d)), lam)
    return dict(Kc=Kc, Vc=Vc, q=q, kn=kn, vn=vn, w_g=w_g, M=M.astype(np.float32), bv=bv.astype(np.float32),
                lens=np.array(lens, np.int32))


def _oracle(c, dtype, append, memory):
    f = lambda x: gen.from_storage(x, dtype)
    Kc, Vc, q = f(c["Kc"]).copy(), f(c["Vc"]).copy(), f(c["q"])
    b, H_q, d = q.shape
    outs, lses = [], []
    for bi in range(b):
        n = int(c["lens"][bi])
        if append:
            Kc[bi, :, n] = f(c["kn"])[bi]
            Vc[bi, :, n] = f(c["vn"])[bi]
            n += 1
        o, lse = im.decode_attention(q[bi], Kc[bi], Vc[bi], n, 1 / math.sqrt(d))
        if memory:
            m, g = im.memory_readout(q[bi], c["M"][bi].astype(np.float64), c["bv"][bi].astype(np.float64),
                                     f(c["w_g"]), 1e-6)
            o = im.residual_output(o, m, g)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses), Kc, Vc


CASES = [
    # dtype, b, H_q, H_kv, d, cap, lens, n_split
    ("bf16", 2, 32, 8, 128, 704, [410, 666], 0),
    ("bf16", 1, 32, 8, 128, 704, [333], 3),
    ("bf16", 3, 32, 8, 128, 304, [0, 17, 303], 5),
    ("bf16", 1, 16, 8, 128, 200, [150], 1),
    ("bf16", 1, 8, 8, 64, 200, [199], 0),
    ("bf16", 2, 64, 8, 128, 504, [257, 300], 7),
    ("bf16", 1, 8, 8, 128, 2152, [2151], 0),
    ("bf16", 1, 32, 8, 128, 64, [0], 2),
    ("f32", 1, 1, 1, 64, 80, [64], 0),
    ("f32", 1, 1, 1, 64, 80, [79], 4),
    ("f32", 2, 8, 2, 128, 96, [33, 60], 2),
    # the 16K workload's 64 (sequence, KV head) pairs with ragged lengths; one split per pair
    ("bf16", 8, 32, 8, 128, 704, [410, 666, 1, 703, 64, 500, 0, 333], 0),
    ("bf16", 1, 64, 8, 128, 2176, [2100], 1),
    ("bf16", 2, 8, 8, 128, 304, [0, 303], 1),
    ("bf16", 3, 16, 8, 128, 64, [1, 63, 32], 1),
]


@pytest.mark.parametrize("dtype,b,H_q,H_kv,d,cap,lens,n_split", CASES)
@pytest.mark.parametrize("append,memory", [(True, True), (False, False), (True, False)])
def test_decode_matches_oracle(dtype, b, H_q, H_kv, d, cap, lens, n_split, append, memory):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, assert_output

    c = _case(dtype, b, H_q, H_kv, d, cap, lens, seed=cap + b + H_q)
    ref_o, ref_lse, ref_K, ref_V = _oracle(c, dtype, append, memory)
    Kc, Vc = to_dev(c["Kc"]), to_dev(np.ascontiguousarray(c["Vc"].transpose(0, 1, 3, 2)))   # V dim-major
    lse = torch.empty((b, H_q), dtype=torch.float32, device=Kc.device)
    o = api.kvm_decode_attn_mem(to_dev(c["q"]), Kc, Vc, to_dev(c["lens"]),
                                k_new=to_dev(c["kn"]) if append else None,
                                v_new=to_dev(c["vn"]) if append else None,
                                M=to_dev(c["M"]) if memory else None, bvec=to_dev(c["bv"]) if memory else None,
                                w_g=to_dev(c["w_g"]) if memory else None, lse=lse, n_split=n_split)
    torch.cuda.synchronize()
    got = to_np(o)
    lse_np = to_np(lse)
    for bi in range(b):
        if lens[bi] == 0 and not append:
            assert np.all(got[bi] == 0) and np.all(np.isneginf(lse_np[bi]))
            continue
        assert_output(got[bi], ref_o[bi], dtype, "o")
        assert_output(lse_np[bi], ref_lse[bi], dtype, "lse")
        # tighter check from the arithmetic: exact inputs, fp32 accumulation
        np.testing.assert_allclose(got[bi], ref_o[bi], rtol=2e-4, atol=2e-4 * np.abs(ref_o[bi]).max())
    if append:
        # the appended rows land in the cache bit-exactly
        gK, gV = to_np(Kc), to_np(Vc)
        for bi in range(b):
            n = lens[bi]
            assert gK[bi, :, n].tobytes() == c["kn"][bi].tobytes()
            assert np.ascontiguousarray(gV[bi, :, :, n]).tobytes() == c["vn"][bi].tobytes()


def test_decode_deterministic_and_split_invariant():
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np

    c = _case("bf16", 2, 32, 8, 128, 904, [800, 899], seed=7)
    outs = []
    for ns in (0, 0, 1, 2, 9, 31):
        Kc, Vc = to_dev(c["Kc"]), to_dev(np.ascontiguousarray(c["Vc"].transpose(0, 1, 3, 2)))
        o = api.kvm_decode_attn_mem(to_dev(c["q"]), Kc, Vc, to_dev(c["lens"]), M=to_dev(c["M"]),
                                    bvec=to_dev(c["bv"]), w_g=to_dev(c["w_g"]), n_split=ns)
        torch.cuda.synchronize()
        outs.append(to_np(o))
    assert outs[0].tobytes() == outs[1].tobytes()
    for x in outs[2:]:
        np.testing.assert_allclose(x, outs[0], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_decode_append_slot_and_full_cache(dtype, d):
    """The new token is attended and written at its slot only when that slot is below the
    attended length: append_slot inside the length replaces that slot's contents, one at
    or past it leaves the cache and the attention alone, and a full cache (len == cap)
    without an append slot drops the token."""
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, assert_output

    cap = 304
    f = lambda x: gen.from_storage(x, dtype)
    for lens, slots in (([300, 200, cap], [100, 250, 5]), ([cap, cap - 1], None)):
        b = len(lens)
        c = _case(dtype, b, 16, 4, d, cap, lens, seed=31 + b)
        Kc, Vc = to_dev(c["Kc"]), to_dev(np.ascontiguousarray(c["Vc"].transpose(0, 1, 3, 2)))
        slot_t = to_dev(np.array(slots, np.int32)) if slots is not None else None
        o = api.kvm_decode_attn_mem(to_dev(c["q"]), Kc, Vc, to_dev(c["lens"]), k_new=to_dev(c["kn"]),
                                    v_new=to_dev(c["vn"]), append_slot=slot_t)
        torch.cuda.synchronize()
        got, gK, gV = to_np(o), to_np(Kc), to_np(Vc)
        for bi in range(b):
            K, V = f(c["Kc"][bi]).copy(), f(c["Vc"][bi]).copy()
            n = min(lens[bi] + (0 if slots is not None else 1), cap)
            app = slots[bi] if slots is not None else lens[bi]
            taken = app < n
            if taken:
                K[:, app] = f(c["kn"])[bi]
                V[:, app] = f(c["vn"])[bi]
            ref, _ = im.decode_attention(f(c["q"])[bi], K, V, n, 1 / math.sqrt(d))
            assert_output(got[bi], ref, dtype, f"o seq {bi}")
            if app < cap:
                want_k = c["kn"][bi] if taken else c["Kc"][bi, :, app]
                want_v = c["vn"][bi] if taken else c["Vc"][bi, :, app]
                assert gK[bi, :, app].tobytes() == np.ascontiguousarray(want_k).tobytes()
                assert np.ascontiguousarray(gV[bi, :, :, app]).tobytes() == np.ascontiguousarray(want_v).tobytes()


def _sweep_cases(n=40):
    """Seeded random decode configurations: group sizes, head dims, dtypes, caps that are
    and are not multiples of 64, lengths from 1 to cap, every append mode, every read-out
    and explicit split counts."""
    r = np.random.default_rng(20261203)
    out = []
    for i in range(n):
        dtype = ["bf16", "f32"][int(r.integers(0, 4) == 0)]
        d = [64, 128][int(r.integers(0, 3) > 0)]
        G = int(r.choice([1, 2, 4, 8]))
        H_kv = int(r.choice([1, 2, 4, 8]))
        b = int(r.integers(1, 4))
        cap = 8 * int(r.integers(1, 90)) if r.random() < 0.6 else 64 * int(r.integers(1, 11))
        mode = ["none", "append", "slot"][int(r.integers(0, 3))]
        lens = [int(r.integers(1, cap + 1)) for _ in range(b)]
        slots = [int(r.integers(0, cap)) for _ in range(b)]
        readout = ["none", "memory", "moments"][int(r.integers(0, 3))]
        n_split = int(r.choice([0, 0, 1, 2, 3, 5, 8, 13]))
        out.append((i, dtype, d, G, H_kv, b, cap, mode, lens, slots, readout, n_split))
    return out


def _pair_cases(n=24):
    """Seeded bf16, d = 128 configurations at the matrix-core path's two extremes: one split
    per (sequence, KV head) (n_split = 1), and the automatic split at 64-80 pairs (the 16K
    workload's batch); every group size, append mode and read-out."""
    r = np.random.default_rng(20261204)
    out = []
    for i in range(n):
        G = int(r.choice([1, 2, 4, 8]))
        auto = i % 2 == 0
        H_kv = 8 if auto else int(r.choice([1, 2, 4, 8]))
        b = int(r.integers(8, 11)) if auto else int(r.integers(1, 4))
        cap = 8 * int(r.integers(1, 90)) if r.random() < 0.6 else 64 * int(r.integers(1, 36))
        mode = ["none", "append", "slot"][int(r.integers(0, 3))]
        lens = [int(r.integers(1, cap + 1)) for _ in range(b)]
        slots = [int(r.integers(0, cap)) for _ in range(b)]
        readout = ["none", "memory", "moments"][int(r.integers(0, 3))]
        out.append((100 + i, "bf16", 128, G, H_kv, b, cap, mode, lens, slots, readout, 0 if auto else 1))
    return out


@pytest.mark.parametrize("case", _sweep_cases() + _pair_cases(),
                         ids=lambda c: f"sweep{c[0]}-{c[1]}-d{c[2]}-G{c[3]}-{c[7]}-{c[10]}")
def test_decode_random_sweep(case):
    import torch
    from oracle import momentkv as mk
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, assert_output

    i, dtype, d, G, H_kv, b, cap, mode, lens, slots, readout, n_split = case
    H_q = G * H_kv
    c = _case(dtype, b, H_q, H_kv, d, cap, lens, seed=1000 + i, n_ev=20)
    f = lambda x: gen.from_storage(x, dtype)
    mom = None
    if readout == "moments":
        rr = gen.rng(93, i, 0, 0)
        moms = [[mk.empty(d) if (bi + g) % 3 == 0 else
                 mk.add(mk.empty(d), f(gen.to_storage(rr.standard_normal((17, d)), dtype)),
                        f(gen.to_storage(rr.standard_normal((17, d)), dtype)))
                 for g in range(H_kv)] for bi in range(b)]
        mom = dict(n_e=to_dev(np.array([[m["n"] for m in row] for row in moms], np.int32)),
                   s_k=to_dev(np.array([[m["sk"] for m in row] for row in moms], np.float32)),
                   s_v=to_dev(np.array([[m["sv"] for m in row] for row in moms], np.float32)),
                   S=to_dev(np.array([[m["S"] for m in row] for row in moms], np.float32)))
    Kc, Vc = to_dev(c["Kc"]), to_dev(np.ascontiguousarray(c["Vc"].transpose(0, 1, 3, 2)))
    lse = torch.empty((b, H_q), dtype=torch.float32, device=Kc.device)
    kw = {}
    if mode != "none":
        kw.update(k_new=to_dev(c["kn"]), v_new=to_dev(c["vn"]))
    if mode == "slot":
        kw.update(append_slot=to_dev(np.array(slots, np.int32)))
    if readout == "memory":
        kw.update(M=to_dev(c["M"]), bvec=to_dev(c["bv"]), w_g=to_dev(c["w_g"]))
    if readout == "moments":
        kw.update(moments=mom)
    o = api.kvm_decode_attn_mem(to_dev(c["q"]), Kc, Vc, to_dev(c["lens"]), lse=lse, n_split=n_split, **kw)
    torch.cuda.synchronize()
    got, glse, gK, gV = to_np(o), to_np(lse), to_np(Kc), to_np(Vc)
    scale = 1 / math.sqrt(d)
    for bi in range(b):
        K, V = f(c["Kc"][bi]).copy(), f(c["Vc"][bi]).copy()
        wantK, wantV = c["Kc"][bi].copy(), c["Vc"][bi].copy()
        if mode == "append":
            n, app = min(lens[bi] + 1, cap), (lens[bi] if lens[bi] < cap else -1)
        elif mode == "slot":
            n = lens[bi]
            app = slots[bi] if slots[bi] < n else -1
        else:
            n, app = lens[bi], -1
        if app >= 0:
            K[:, app], V[:, app] = f(c["kn"])[bi], f(c["vn"])[bi]
            wantK[:, app], wantV[:, app] = c["kn"][bi], c["vn"][bi]
        ref, ref_lse = im.decode_attention(f(c["q"])[bi], K, V, n, scale)
        if readout == "memory":
            m, g = im.memory_readout(f(c["q"])[bi], c["M"][bi].astype(np.float64), c["bv"][bi].astype(np.float64),
                                     f(c["w_g"]), 1e-6)
            ref = im.residual_output(ref, m, g)
        elif readout == "moments":
            qd = f(c["q"])[bi]
            for h in range(H_q):
                m32 = {k: (np.float32(v).astype(np.float64) if k != "n" else v) for k, v in moms[bi][h // G].items()}
                ref[h] = mk.mix(qd[h], ref[h], float(ref_lse[h]), m32, d)[0]
        assert_output(got[bi], ref, dtype, f"o seq {bi}")
        np.testing.assert_allclose(got[bi], ref, rtol=1e-3, atol=1e-3 * np.abs(ref).max())
        np.testing.assert_allclose(glse[bi], ref_lse, rtol=1e-4, atol=1e-4)
        # the caches change at the new token's slot only
        assert gK[bi].tobytes() == wantK.tobytes()
        assert gV[bi].tobytes() == np.ascontiguousarray(wantV.transpose(0, 2, 1)).tobytes()


PROJ_CASES = [
    # dtype, b, H_q, H_kv, d, cap, lens, n_split
    ("bf16", 2, 32, 8, 128, 704, [410, 666], 0),     # matrix-core path
    ("bf16", 1, 16, 2, 64, 200, [150], 3),           # d 64, group of 8
    ("f32", 2, 8, 2, 128, 96, [33, 60], 2),          # FMA path
    ("bf16", 8, 32, 8, 128, 704, [410, 666, 1, 703, 64, 500, 7, 333], 0),   # 64 pairs
    ("bf16", 1, 64, 8, 128, 304, [300], 1),          # one split, group of 8
]


@pytest.mark.parametrize("dtype,b,H_q,H_kv,d,cap,lens,n_split", PROJ_CASES)
def test_readout_projection_matches_oracle(dtype, b, H_q, H_kv, d, cap, lens, n_split):
    """kvm_mem_query against the oracle's W_m q, and the decode read-out addressed with the
    projected query.  The decode check feeds both sides the oracle's projected query
    (rounded to the storage type), so only the read-out arithmetic is compared; the
    pipeline check (the GPU's own projection into the decode) takes the output bar."""
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, assert_output

    c = _case(dtype, b, H_q, H_kv, d, cap, lens, seed=cap + 7)
    r = gen.rng(92, d, H_q, 0)
    W_m = gen.to_storage(np.eye(d) + r.standard_normal((d, d)) / math.sqrt(d), dtype)
    f = lambda x: gen.from_storage(x, dtype)
    qd = f(c["q"])
    qm_ref = np.stack([im.memory_query(qd[i], f(W_m)) for i in range(b)])
    # the projection: fp32 accumulation, then one rounding to the storage type
    got_qm = f(to_np(api.kvm_mem_query(to_dev(c["q"]), to_dev(W_m))))
    ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -22
    np.testing.assert_allclose(got_qm, qm_ref, rtol=ulp, atol=1e-6 * np.abs(qm_ref).max())

    qm_st = gen.to_storage(qm_ref, dtype)
    Kc, Vc = to_dev(c["Kc"]), to_dev(np.ascontiguousarray(c["Vc"].transpose(0, 1, 3, 2)))
    o = to_np(api.kvm_decode_attn_mem(to_dev(c["q"]), Kc, Vc, to_dev(c["lens"]), k_new=to_dev(c["kn"]),
                                      v_new=to_dev(c["vn"]), M=to_dev(c["M"]), bvec=to_dev(c["bv"]),
                                      w_g=to_dev(c["w_g"]), n_split=n_split, q_mem=to_dev(qm_st)))
    Kr, Vr = f(c["Kc"]).copy(), f(c["Vc"]).copy()
    for i in range(b):
        n = int(c["lens"][i])
        Kr[i, :, n], Vr[i, :, n] = f(c["kn"])[i], f(c["vn"])[i]
        oa, _ = im.decode_attention(qd[i], Kr[i], Vr[i], n + 1, 1 / math.sqrt(d))
        m, g = im.memory_readout(qd[i], c["M"][i].astype(np.float64), c["bv"][i].astype(np.float64), f(c["w_g"]),
                                 1e-6, q_mem=f(qm_st)[i])
        ref = im.residual_output(oa, m, g)
        assert_output(o[i], ref, dtype, f"seq {i}: o with the projected query")
        np.testing.assert_allclose(o[i], ref, rtol=2e-4, atol=2e-4 * np.abs(ref).max())
        # the projection changes the output: the unprojected read-out is far from it
        m0, g0 = im.memory_readout(qd[i], c["M"][i].astype(np.float64), c["bv"][i].astype(np.float64), f(c["w_g"]))
        assert np.abs(im.residual_output(oa, m0, g0) - ref).max() > 1e-3 * np.abs(ref).max()

    # pipeline: the GPU's projection feeds the GPU decode (fresh caches: the call above
    # wrote the new token)
    Kc, Vc = to_dev(c["Kc"]), to_dev(np.ascontiguousarray(c["Vc"].transpose(0, 1, 3, 2)))
    qm_dev = api.kvm_mem_query(to_dev(c["q"]), to_dev(W_m))
    o2 = to_np(api.kvm_decode_attn_mem(to_dev(c["q"]), Kc, Vc, to_dev(c["lens"]), k_new=to_dev(c["kn"]),
                                       v_new=to_dev(c["vn"]), M=to_dev(c["M"]), bvec=to_dev(c["bv"]),
                                       w_g=to_dev(c["w_g"]), n_split=n_split, q_mem=qm_dev))
    for i in range(b):
        n = int(c["lens"][i])
        oa, _ = im.decode_attention(qd[i], Kr[i], Vr[i], n + 1, 1 / math.sqrt(d))
        m, g = im.memory_readout(qd[i], c["M"][i].astype(np.float64), c["bv"][i].astype(np.float64), f(c["w_g"]),
                                 1e-6, q_mem=qm_ref[i])
        assert_output(o2[i], im.residual_output(oa, m, g), dtype, f"seq {i}: projection pipeline")


def _merge_stress_inputs(r, layers, steps, b, H_q, H_kv, d, cap, lens):
    st = lambda x: gen.to_storage(x, "bf16")
    Ls = []
    for _ in range(layers):
        M = np.zeros((b, H_kv, d, d))
        bv = np.zeros((b, H_kv, d))
        for bi in range(b):
            for g in range(H_kv):
                M[bi, g], bv[bi, g] = im.memory_build(r.standard_normal((30, d)), r.standard_normal((30, d)), 0.99)
        Ls.append(dict(Kc=st(r.standard_normal((b, H_kv, cap, d))), Vc=st(r.standard_normal((b, H_kv, cap, d))),
                       w_g=st(r.standard_normal((H_q, d)) / math.sqrt(d)), M=M.astype(np.float32),
                       bv=bv.astype(np.float32),
                       q=st(r.standard_normal((steps, b, H_q, d))), kn=st(r.standard_normal((steps, b, H_kv, d))),
                       vn=st(r.standard_normal((steps, b, H_kv, d)))))
    return Ls


def _merge_stress_ref(Ls, l, t, lens, d):
    """Oracle output of layer l at step t: caches grown by steps 0..t, memory read-out."""
    f = lambda x: gen.from_storage(x, "bf16")
    c = Ls[l]
    out = []
    for bi in range(len(lens)):
        K, V = f(c["Kc"][bi]).copy(), f(c["Vc"][bi]).copy()
        for u in range(t + 1):
            K[:, lens[bi] + u], V[:, lens[bi] + u] = f(c["kn"][u, bi]), f(c["vn"][u, bi])
        o, _ = im.decode_attention(f(c["q"][t, bi]), K, V, lens[bi] + t + 1, 1 / math.sqrt(d))
        m, g = im.memory_readout(f(c["q"][t, bi]), c["M"][bi].astype(np.float64), c["bv"][bi].astype(np.float64),
                                 f(c["w_g"]), 1e-6)
        out.append(im.residual_output(o, m, g))
    return np.stack(out)


def test_decode_many_launches_and_graph_replays():
    """Back-to-back decode launches at the 16K workload's decode shape (batch 8, 32/8 heads,
    ~1900 slots), two layers sharing one workspace, new inputs every step: every launch's
    output must match the oracle (a merge reading block states left by an earlier launch
    would not), eagerly and replayed from a HIP graph with fresh inputs copied in between
    replays."""
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, assert_output

    b, H_q, H_kv, d, layers, steps = 8, 32, 8, 128, 2, 12
    cap = api.cache_cap(1900 + steps)
    r = gen.rng(94, 0, 0, 0)
    lens = [1880 + 3 * i for i in range(b)]
    Ls = _merge_stress_inputs(r, layers, steps, b, H_q, H_kv, d, cap, lens)
    ws = torch.zeros(8 << 20, dtype=torch.uint8, device="cuda")
    D = []
    for c in Ls:
        D.append(dict(Kc=to_dev(c["Kc"]), Vc=to_dev(np.ascontiguousarray(c["Vc"].transpose(0, 1, 3, 2))),
                      M=to_dev(c["M"]), bv=to_dev(c["bv"]), w_g=to_dev(c["w_g"])))
    lens_t = to_dev(np.array(lens, np.int32))
    outs = [[None] * steps for _ in range(layers)]
    # eager: steps 0 .. steps/2 - 1
    half = steps // 2
    for t in range(half):
        for l in range(layers):
            c = Ls[l]
            outs[l][t] = api.kvm_decode_attn_mem(to_dev(c["q"][t]), D[l]["Kc"], D[l]["Vc"], lens_t,
                                                 k_new=to_dev(c["kn"][t]), v_new=to_dev(c["vn"][t]), M=D[l]["M"],
                                                 bvec=D[l]["bv"], w_g=D[l]["w_g"], ws=ws)
        api.kvm_len_add(lens_t, 1)
    torch.cuda.synchronize()
    # graph: one step of both layers captured over static input buffers, replayed with the
    # remaining steps' inputs copied in
    qb = [torch.empty((b, H_q, d), dtype=torch.bfloat16, device=lens_t.device) for _ in range(layers)]
    kb = [torch.empty((b, H_kv, d), dtype=torch.bfloat16, device=lens_t.device) for _ in range(layers)]
    vb = [torch.empty((b, H_kv, d), dtype=torch.bfloat16, device=lens_t.device) for _ in range(layers)]
    ob = [torch.empty((b, H_q, d), dtype=torch.float32, device=lens_t.device) for _ in range(layers)]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for l in range(layers):
                api.kvm_decode_attn_mem(qb[l], D[l]["Kc"], D[l]["Vc"], lens_t, k_new=kb[l], v_new=vb[l], M=D[l]["M"],
                                        bvec=D[l]["bv"], w_g=D[l]["w_g"], o=ob[l], ws=ws, stream=stream)
            api.kvm_len_add(lens_t, 1, stream=stream)
    torch.cuda.synchronize()
    # capture launched nothing: the caches and lengths still stand after the eager steps
    assert to_np(lens_t).tolist() == [x + half for x in lens]
    for t in range(half, steps):
        for l in range(layers):
            c = Ls[l]
            qb[l].copy_(to_dev(c["q"][t]))
            kb[l].copy_(to_dev(c["kn"][t]))
            vb[l].copy_(to_dev(c["vn"][t]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(layers):
            outs[l][t] = ob[l].clone()
    torch.cuda.synchronize()
    for l in range(layers):
        for t in range(steps):
            ref = _merge_stress_ref(Ls, l, t, lens, d)
            got = to_np(outs[l][t])
            for bi in range(b):
                assert_output(got[bi], ref[bi], "bf16", f"layer {l} step {t} seq {bi}")
                np.testing.assert_allclose(got[bi], ref[bi], rtol=2e-4, atol=2e-4 * np.abs(ref[bi]).max(),
                                           err_msg=f"layer {l} step {t} seq {bi}")
