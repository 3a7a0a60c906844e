"""Pre-eviction top-k (bit-exact), compaction (bit-exact) and the fused memory / moment
build against the oracle."""
import math

import numpy as np
import pytest

from oracle import indexmem as im
from oracle import momentkv as mk
from synth import gen

pytestmark = pytest.mark.gpu


def _scores(rows, L, seed, ties=0, specials=False):
    s = gen.make_scores(7, rows, L, seed, ties)
    if specials and L >= 8:
        r = gen.rng(7, 1, 0, seed)
        for row in range(rows):
            pos = r.choice(L, size=min(L, 6), replace=False)
            s[row, pos[0]] = np.nan
            s[row, pos[1]] = -0.0
            s[row, pos[2]] = 0.0
            s[row, pos[3]] = -np.inf
            s[row, pos[4]] = np.inf
    return s


TOPK = [  # rows, L, B, R, inclusive, ties, specials
    (1, 1, 1, 0, True, 0, False),
    (3, 5, 2, 1, True, 2, False),
    (2, 512, 64, 0, True, 0, True),
    (1, 4096, 410, 32, True, 0, False),
    (8, 16384, 1638, 32, True, 0, False),
    (8, 16384, 1638, 32, True, 3, True),
    (1, 131072, 1024, 64, False, 0, False),
    (32, 32768, 128, 0, True, 0, False),
    (4, 3000, 3000, 0, True, 0, False),   # keep all
    (4, 3000, 7, 7, True, 0, False),      # recent window only
    (2, 1025, 1024, 64, False, 50, True),  # more slots than candidates
    # rows longer than 32768 positions take the many-blocks-per-row path with a workspace
    (3, 40000, 999, 13, True, 0, True),   # ragged last chunk, specials
    (2, 36000, 36000, 0, True, 0, False),  # keep all
    (2, 36000, 16, 16, True, 0, False),   # recent window only
    (1, 40000, 4000, 64, False, 2, False),  # long runs of equal keys across chunk boundaries
    (2, 50000, 300, 0, True, 0, False),   # scores spread over many binades (three levels)
    # the register-resident path's boundaries (rows of at most 4096 / 16384 positions) and the
    # one-block path just past them
    (2, 4097, 400, 16, True, 5, True),
    (1, 16385, 1600, 32, True, 0, True),
    (4, 4096, 4000, 0, True, 2, False),   # nearly everything kept, ties
    (2, 16384, 16000, 100, False, 7, True),
    (3, 16384, 1, 0, True, 0, False),     # k = 1
    (2, 12000, 300, 0, True, 0, False),   # many binades in registers (three levels)
]


@pytest.mark.parametrize("rows,L,B,R,inc,ties,specials", TOPK)
@pytest.mark.parametrize("one_block", [False, True], ids=["wide", "one_block"])
def test_topk_bit_exact(rows, L, B, R, inc, ties, specials, one_block):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np
    I = _scores(rows, L, seed=L + B, ties=ties, specials=specials)
    if (L, B) in ((50000, 300), (12000, 300)):
        # magnitudes from 1e-30 to 1e30, both signs: a key span that needs three 12-bit levels
        r = gen.rng(7, 2, 0, 0)
        I = (np.sign(r.standard_normal((rows, L))) * 10.0 ** r.uniform(-30, 30, (rows, L))).astype(np.float32)
    # a workspace holding garbage: the result must not depend on its contents
    ws = torch.full((1 << 22,), 0x5a, dtype=torch.uint8, device="cuda")
    idx, sm = api.kvm_topk_select(to_dev(I), B, R, inc, ws=None if one_block else ws, one_block=one_block)
    torch.cuda.synchronize()
    gi, gs = to_np(idx), to_np(sm)
    for r in range(rows):
        ri, rs = im.topk_select(I[r].astype(np.float64), B, R, inc)
        assert gi[r].tolist() == ri.tolist(), f"row {r}"
        assert gs[r].tolist() == rs.tolist(), f"row {r}"


@pytest.mark.parametrize("L", [100, 4096, 16384, 20000, 40000])
@pytest.mark.parametrize("value", [1.0, -np.inf, np.nan])
def test_topk_all_scores_equal(L, value):
    """Every candidate key equal (a zero key span: no histogram pass): the kept ones are the
    lowest positions, on every path (registers, one block, many blocks)."""
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np
    I = np.full((2, L), value, np.float32)
    ws = torch.full((1 << 22,), 0x5a, dtype=torch.uint8, device="cuda")
    for one_block in (False, True):
        idx, sm = api.kvm_topk_select(to_dev(I), 50, 3, True, ws=None if one_block else ws, one_block=one_block)
        torch.cuda.synchronize()
        gi, gs = to_np(idx), to_np(sm)
        for r in range(2):
            ri, rs = im.topk_select(I[r].astype(np.float64), 50, 3, True)
            assert gi[r].tolist() == ri.tolist() and gs[r].tolist() == rs.tolist(), (one_block, r)


def _kv(dtype, b, L, H, d, seed):
    r = gen.rng(91, seed, 0, 0)
    return (gen.to_storage(r.standard_normal((b, L, H, d)), dtype),
            gen.to_storage(r.standard_normal((b, L, H, d)), dtype))


COMPACT = [  # dtype, b, L, H_kv, d, B, R, lam, cap_extra
    ("bf16", 1, 4096, 8, 128, 410, 32, 0.995, 256),
    ("bf16", 2, 1000, 2, 128, 100, 7, 0.995, 3),
    ("bf16", 1, 3001, 3, 64, 200, 0, 0.99, 0),
    ("bf16", 1, 700, 2, 128, 50, 0, 1.0, 0),
    ("bf16", 1, 700, 2, 128, 50, 0, 0.0, 0),
    ("bf16", 1, 40, 1, 128, 40, 0, 0.9, 0),   # nothing evicted
    ("f32", 1, 512, 1, 64, 64, 0, 0.99, 16),
    ("f32", 2, 333, 2, 128, 30, 5, 0.9, 0),
]


@pytest.mark.parametrize("dtype,b,L,H,d,B,R,lam,extra", COMPACT)
def test_compact_and_memory_build(dtype, b, L, H, d, B, R, lam, extra):
    import torch
    lam = float(np.float32(lam))      # the library takes lambda as fp32: both sides use that value
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, assert_output, normwise, maxabs
    Kt, Vt = _kv(dtype, b, L, H, d, seed=L + d)
    I = _scores(b, L, seed=L)
    sel = [im.topk_select(I[i].astype(np.float64), B, R) for i in range(b)]
    smaps = [x[1] for x in sel]
    idxs = np.stack([x[0] for x in sel]).astype(np.int32)
    keep = L - int((smaps[0] < 0).sum())
    cap = keep + extra
    rM = gen.rng(92, L, 0, 0)
    M0 = rM.standard_normal((b, H, d, d)).astype(np.float32)
    b0 = np.abs(rM.standard_normal((b, H, d))).astype(np.float32)
    M = to_dev(M0.copy())
    bv = to_dev(b0.copy())
    Kc, Vc = api.kvm_compact_kv(to_dev(Kt), to_dev(Vt), to_dev(np.stack(smaps).astype(np.int32)), to_dev(idxs), keep, cap,
                                M=M, bvec=bv, lam=lam)
    torch.cuda.synchronize()
    gK, gV, gM, gb = to_np(Kc), to_np(Vc), to_np(M), to_np(bv)
    Kd, Vd = gen.from_storage(Kt, dtype), gen.from_storage(Vt, dtype)
    for i in range(b):
        rK, rV = im.compact(Kt[i], Vt[i], smaps[i], cap)
        assert gK[i].tobytes() == rK.tobytes()
        assert gV[i].tobytes() == np.ascontiguousarray(rV.transpose(0, 2, 1)).tobytes()   # V dim-major
        ev = im.evicted_in_order(smaps[i])
        for g in range(H):
            refM, refb = im.memory_build(Kd[i, ev, g], Vd[i, ev, g], lam, M0[i, g], b0[i, g])
            assert_output(gM[i, g], refM, dtype, "M")
            assert_output(gb[i, g], refb, dtype, "b")
            if dtype == "bf16":
                # hi+lo split keeps ~16 bits of lam^(n-i) phi(k): far inside the bar
                assert normwise(gM[i, g], refM) < 1e-4
                assert normwise(gb[i, g], refb) < 1e-5


@pytest.mark.parametrize("head_major", [False, True])
def test_moment_update_per_head(head_major):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise
    b, L, H, d, keep = 2, 2000, 4, 128, 999
    Kt, Vt = _kv("bf16", b, L, H, d, seed=5)
    if head_major:
        Kt, Vt = np.ascontiguousarray(Kt.transpose(0, 2, 1, 3)), np.ascontiguousarray(Vt.transpose(0, 2, 1, 3))
    I = _scores(b * H, L, seed=9)
    sel = [im.topk_select(I[r].astype(np.float64), keep, 0) for r in range(b * H)]
    smaps = np.stack([x[1] for x in sel]).astype(np.int32)
    idxs = np.stack([x[0] for x in sel]).astype(np.int32)
    r0 = gen.rng(93, 0, 0, 0)
    n0 = np.full((b, H), 17, np.int32)
    sk0, sv0 = r0.standard_normal((b, H, d)).astype(np.float32), r0.standard_normal((b, H, d)).astype(np.float32)
    S0 = r0.standard_normal((b, H, d, d)).astype(np.float32)
    mom = dict(n_e=to_dev(n0.copy()), s_k=to_dev(sk0.copy()), s_v=to_dev(sv0.copy()), S=to_dev(S0.copy()))
    Kc, Vc = api.kvm_compact_kv(to_dev(Kt), to_dev(Vt), to_dev(smaps), to_dev(idxs), keep, keep + 5, moments=mom,
                                per_head=True, kv_head_major=head_major)
    torch.cuda.synchronize()
    Kd, Vd = gen.from_storage(Kt, "bf16"), gen.from_storage(Vt, "bf16")
    gK = to_np(Kc)
    for i in range(b):
        for g in range(H):
            sm = smaps[i * H + g]
            kk = Kd[i, g] if head_major else Kd[i, :, g]
            vv = Vd[i, g] if head_major else Vd[i, :, g]
            ev = np.nonzero(sm < 0)[0]
            m = dict(n=17, sk=sk0[i, g].astype(np.float64), sv=sv0[i, g].astype(np.float64),
                     S=S0[i, g].astype(np.float64))
            m = mk.add(m, kk[ev], vv[ev])
            assert int(to_np(mom["n_e"])[i, g]) == m["n"]
            assert normwise(to_np(mom["S"])[i, g], m["S"]) < 1e-5
            assert normwise(to_np(mom["s_k"])[i, g], m["sk"]) < 1e-5
            assert normwise(to_np(mom["s_v"])[i, g], m["sv"]) < 1e-5
            kept = np.nonzero(sm >= 0)[0]
            src = (Kt[i, g] if head_major else Kt[i, :, g])[kept]
            assert gK[i, g, :keep].tobytes() == src.tobytes()


def test_gather_rows_and_rank_r_update():
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise
    rows, L, E = 3, 777, 64
    src = gen.rng(94, 0, 0, 0).standard_normal((rows, L, E)).astype(np.float32)
    I = _scores(rows, L, seed=3)
    smaps = np.stack([im.topk_select(I[r].astype(np.float64), 70, 6)[1] for r in range(rows)]).astype(np.int32)
    dst = api.kvm_gather_rows(to_dev(src), to_dev(smaps), 80)
    torch.cuda.synchronize()
    got = to_np(dst)
    for r in range(rows):
        kept = np.nonzero(smaps[r] >= 0)[0]
        assert got[r, :len(kept)].tobytes() == src[r, kept].tobytes()
        assert not got[r, len(kept):].any()
    # rank-r decayed update == sequential recurrence
    b, rr, H, d, lam = 2, 37, 3, 128, float(np.float32(0.97))
    rg = gen.rng(95, 0, 0, 0)
    Kr = gen.to_storage(rg.standard_normal((b, rr, H, d)), "bf16")
    Vr = gen.to_storage(rg.standard_normal((b, rr, H, d)), "bf16")
    M0 = rg.standard_normal((b, H, d, d)).astype(np.float32)
    b0 = rg.standard_normal((b, H, d)).astype(np.float32)
    M, bv = to_dev(M0.copy()), to_dev(b0.copy())
    api.kvm_mem_update(to_dev(Kr), to_dev(Vr), M, bv, lam)
    torch.cuda.synchronize()
    Kd, Vd = gen.from_storage(Kr, "bf16"), gen.from_storage(Vr, "bf16")
    for i in range(b):
        for g in range(H):
            rM, rb = im.memory_update_sequential(Kd[i, :, g], Vd[i, :, g], lam, M0[i, g], b0[i, g])
            assert normwise(to_np(M)[i, g], rM) < 1e-5
            assert normwise(to_np(bv)[i, g], rb) < 1e-5
    # single row taken from the cache at a device-given slot
    cap = 16
    Kc = gen.to_storage(rg.standard_normal((b, H, cap, d)), "bf16")
    Vc = gen.to_storage(rg.standard_normal((b, H, cap, d)), "bf16")
    slots = np.array([3, 10], np.int32)
    M, bv = to_dev(M0.copy()), to_dev(b0.copy())
    api.kvm_mem_update(to_dev(Kc), to_dev(np.ascontiguousarray(Vc.transpose(0, 1, 3, 2))), M, bv, lam,
                       row_slot=to_dev(slots))
    torch.cuda.synchronize()
    Kd, Vd = gen.from_storage(Kc, "bf16"), gen.from_storage(Vc, "bf16")
    for i in range(b):
        for g in range(H):
            rM, rb = im.memory_update_sequential(Kd[i, g, slots[i]][None], Vd[i, g, slots[i]][None], lam,
                                                 M0[i, g], b0[i, g])
            assert normwise(to_np(M)[i, g], rM) < 1e-5
            assert normwise(to_np(bv)[i, g], rb) < 1e-5



@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
def test_moment_update_matches_oracle(dt, d):
    """kvm_moment_update: rows folded into the moment sums of each (sequence, KV head)
    [MKV part 1], against the oracle's running sums; then one row per sequence taken from
    the caches at a device-given slot (a slot outside the cache leaves the sums as they are)."""
    import torch
    from oracle import momentkv as mk
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise
    b, rr, H = 3, 45, 2
    rg = gen.rng(96, d, 0, 0)
    Kr = gen.to_storage(rg.standard_normal((b, rr, H, d)), dt)
    Vr = gen.to_storage(rg.standard_normal((b, rr, H, d)), dt)
    n0 = rg.integers(0, 50, (b, H)).astype(np.int32)
    sk0 = rg.standard_normal((b, H, d)).astype(np.float32)
    sv0 = rg.standard_normal((b, H, d)).astype(np.float32)
    S0 = rg.standard_normal((b, H, d, d)).astype(np.float32)
    mom = dict(n_e=to_dev(n0.copy()), s_k=to_dev(sk0.copy()), s_v=to_dev(sv0.copy()), S=to_dev(S0.copy()))
    api.kvm_moment_update(to_dev(Kr), to_dev(Vr), mom)
    torch.cuda.synchronize()
    Kd, Vd = gen.from_storage(Kr, dt), gen.from_storage(Vr, dt)
    got = {k: to_np(v) for k, v in mom.items()}
    for i in range(b):
        for g in range(H):
            ref = mk.add(dict(n=int(n0[i, g]), sk=sk0[i, g], sv=sv0[i, g], S=S0[i, g]), Kd[i, :, g], Vd[i, :, g])
            assert got["n_e"][i, g] == ref["n"]
            assert normwise(got["s_k"][i, g], ref["sk"]) < 1e-6
            assert normwise(got["s_v"][i, g], ref["sv"]) < 1e-6
            assert normwise(got["S"][i, g], ref["S"]) < 1e-6
    cap = 24
    Kc = gen.to_storage(rg.standard_normal((b, H, cap, d)), dt)
    Vc = gen.to_storage(rg.standard_normal((b, H, cap, d)), dt)
    slots = np.array([5, cap, 17], np.int32)   # the second sequence: no row
    mom = dict(n_e=to_dev(n0.copy()), s_k=to_dev(sk0.copy()), s_v=to_dev(sv0.copy()), S=to_dev(S0.copy()))
    api.kvm_moment_update(to_dev(Kc), to_dev(np.ascontiguousarray(Vc.transpose(0, 1, 3, 2))), mom,
                          row_slot=to_dev(slots))
    torch.cuda.synchronize()
    Kd, Vd = gen.from_storage(Kc, dt), gen.from_storage(Vc, dt)
    got = {k: to_np(v) for k, v in mom.items()}
    for i in range(b):
        for g in range(H):
            m0 = dict(n=int(n0[i, g]), sk=sk0[i, g], sv=sv0[i, g], S=S0[i, g])
            ref = m0 if slots[i] >= cap else mk.add(m0, Kd[i, g, slots[i]][None], Vd[i, g, slots[i]][None])
            assert got["n_e"][i, g] == ref["n"]
            assert normwise(got["s_k"][i, g], ref["sk"]) < 1e-6
            assert normwise(got["s_v"][i, g], ref["sv"]) < 1e-6
            assert normwise(got["S"][i, g], ref["S"]) < 1e-6

def _compact_sweep(n=24):
    """Seeded random shapes for the top-k + compaction + memory build chain."""
    r = np.random.default_rng(777)
    out = []
    for i in range(n):
        dtype = "bf16" if r.random() < 0.75 else "f32"
        d = int(r.choice([64, 128]))
        b, H = int(r.integers(1, 3)), int(r.integers(1, 5))
        L = int(r.integers(33, 3000))
        B = int(r.integers(1, L + 1))
        R = int(r.integers(0, min(B, 40) + 1))
        lam = float(r.choice([0.0, 0.5, 0.9, 0.99, 1.0]))
        extra = int(r.integers(0, 100))
        out.append((i, dtype, b, L, H, d, B, R, lam, extra))
    return out


@pytest.mark.parametrize("case", _compact_sweep(), ids=lambda c: f"sweep{c[0]}-{c[1]}-L{c[3]}-d{c[5]}")
def test_select_compact_build_random_sweep(case):
    """top-k (bit-exact), compaction (bit-exact) and the memory build (the bar) on random
    shapes, each step fed by the GPU's previous one only where the oracle agrees exactly."""
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, assert_output
    i, dtype, b, L, H, d, B, R, lam, extra = case
    lam = float(np.float32(lam))
    I = _scores(b, L, seed=5000 + i, ties=int(i % 3), specials=(i % 4 == 0))
    idx, sm = api.kvm_topk_select(to_dev(I), B, R)
    torch.cuda.synchronize()
    gi, gs = to_np(idx), to_np(sm)
    sel = [im.topk_select(I[r].astype(np.float64), B, R) for r in range(b)]
    for r in range(b):
        assert gi[r].tolist() == sel[r][0].tolist() and gs[r].tolist() == sel[r][1].tolist(), f"row {r}"
    keep = gi.shape[1]
    cap = keep + extra
    Kt, Vt = _kv(dtype, b, L, H, d, seed=6000 + i)
    rM = gen.rng(94, i, 0, 0)
    M0 = rM.standard_normal((b, H, d, d)).astype(np.float32)
    b0 = np.abs(rM.standard_normal((b, H, d))).astype(np.float32)
    M, bv = to_dev(M0.copy()), to_dev(b0.copy())
    Kc, Vc = api.kvm_compact_kv(to_dev(Kt), to_dev(Vt), sm, idx, keep, cap, M=M, bvec=bv, lam=lam)
    torch.cuda.synchronize()
    gK, gV, gM, gb = to_np(Kc), to_np(Vc), to_np(M), to_np(bv)
    Kd, Vd = gen.from_storage(Kt, dtype), gen.from_storage(Vt, dtype)
    for r in range(b):
        rK, rV = im.compact(Kt[r], Vt[r], sel[r][1], cap)
        assert gK[r][:, :keep].tobytes() == np.ascontiguousarray(rK[:, :keep]).tobytes()
        assert np.ascontiguousarray(gV[r][:, :, :keep]).tobytes() == \
            np.ascontiguousarray(rV[:, :keep].transpose(0, 2, 1)).tobytes()
        ev = im.evicted_in_order(sel[r][1])
        for g in range(H):
            refM, refb = im.memory_build(Kd[r, ev, g], Vd[r, ev, g], lam, M0[r, g], b0[r, g])
            assert_output(gM[r, g], refM, dtype, f"M seq {r} head {g}")
            assert_output(gb[r, g], refb, dtype, f"b seq {r} head {g}")
