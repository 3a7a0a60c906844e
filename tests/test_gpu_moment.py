"""MomentKV on the GPU against the oracle: the attention weight alpha (two matrix-core
passes), the residual score, the stand-alone read-out, and the whole moment-informed
prefill (halving rounds of score -> per-head top-k -> moment fold) followed by decode
with the normalization-corrected mix."""
import math

import numpy as np
import pytest

from oracle import indexmem as im
from oracle import momentkv as mk
from synth import WORKLOADS, gen

pytestmark = pytest.mark.gpu


def _qkv(b, L, W, H_q, H_kv, d, seed):
    r = gen.rng(95, seed, 0, 0)
    st = lambda x: gen.to_storage(x, "bf16")
    return st(r.standard_normal((b, W, H_q, d))), st(r.standard_normal((b, L, H_kv, d))), \
        st(r.standard_normal((b, L, H_kv, d)))


ALPHA_CASES = [
    # b, L, W, H_q, H_kv, d, head_major
    (2, 1000, 64, 32, 8, 128, False),
    (1, 777, 64, 32, 8, 128, True),
    (1, 531, 32, 8, 8, 64, False),
    (2, 64, 64, 16, 4, 128, False),      # every key inside the window
    (1, 2048, 16, 4, 2, 64, True),
]


@pytest.mark.parametrize("b,L,W,H_q,H_kv,d,hm", ALPHA_CASES)
def test_alpha_matches_oracle(b, L, W, H_q, H_kv, d, hm):
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise
    Q, Kt, _ = _qkv(b, L, W, H_q, H_kv, d, seed=L + W)
    Kin = np.ascontiguousarray(Kt.transpose(0, 2, 1, 3)) if hm else Kt
    got = to_np(api.kvm_moment_alpha(to_dev(Q), to_dev(Kin), kv_head_major=hm))
    Qd, Kd = gen.from_storage(Q, "bf16"), gen.from_storage(Kt, "bf16")
    for i in range(b):
        ref = mk.alpha(Qd[i], Kd[i], np.arange(L - W, L), 1 / math.sqrt(d), H_q // H_kv)
        assert normwise(got[i], ref) < 1e-5
        np.testing.assert_allclose(got[i], ref, rtol=1e-4, atol=1e-6 * ref.max())
        # each query's weights sum to one, so alpha sums to 1 per KV head
        np.testing.assert_allclose(got[i].sum(-1), 1.0, rtol=1e-4)


def _moments(b, H, d, n, seed):
    """Moments of n random evicted rows per (sequence, KV head), in fp64 and as device
    arrays (n = 0 gives empty moments)."""
    r = gen.rng(96, seed, 0, 0)
    moms = []
    for i in range(b):
        row = []
        for g in range(H):
            m = mk.empty(d)
            if n:
                m = mk.add(m, gen.bf16_to_f32(gen.to_storage(r.standard_normal((n, d)), "bf16")),
                           gen.bf16_to_f32(gen.to_storage(r.standard_normal((n, d)), "bf16")))
            row.append(m)
        moms.append(row)
    return moms


def _dev_moments(moms):
    from tests.gpu_util import to_dev
    return dict(n_e=to_dev(np.array([[m["n"] for m in row] for row in moms], np.int32)),
                s_k=to_dev(np.array([[m["sk"] for m in row] for row in moms], np.float32)),
                s_v=to_dev(np.array([[m["sv"] for m in row] for row in moms], np.float32)),
                S=to_dev(np.array([[m["S"] for m in row] for row in moms], np.float32)))


@pytest.mark.parametrize("L,d,n,hm", [(1000, 128, 300, False), (513, 64, 50, True), (300, 128, 0, False),
                                      (4097, 128, 4000, True),
                                      # a last block of 3 tiles: the tile ring's loop without a tail
                                      (864, 128, 100, False), (352, 64, 20, True),
                                      # >= 256 blocks of 1024 keys: the wide-block variant
                                      (32769, 128, 5000, False), (32000, 64, 100, True)])
def test_residual_score_matches_oracle(L, d, n, hm):
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, normwise
    b, H = 2, 4
    _, Kt, Vt = _qkv(b, L, 1, 1, H, d, seed=L + n)
    moms = _moments(b, H, d, n, seed=L)
    alpha = gen.rng(97, L, 0, 0).random((b, H, L)).astype(np.float32)
    tr = (lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))) if hm else (lambda x: x)
    mom_d = _dev_moments(moms)
    got = to_np(api.kvm_moment_score(to_dev(tr(Kt)), to_dev(tr(Vt)), to_dev(alpha), mom_d, kv_head_major=hm))
    Kd, Vd = gen.from_storage(Kt, "bf16"), gen.from_storage(Vt, "bf16")
    for i in range(b):
        for g in range(H):
            m32 = {k: (np.float32(v).astype(np.float64) if k != "n" else v) for k, v in moms[i][g].items()}
            ref = mk.score(alpha[i, g].astype(np.float64), Kd[i, :, g], Vd[i, :, g], m32, d)
            assert normwise(got[i, g], ref) < 1e-5
            np.testing.assert_allclose(got[i, g], ref, rtol=2e-5, atol=1e-6 * np.abs(ref).max())


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f32", 1), ("bf16", 8)])
def test_moment_readout_matches_oracle(dtype, G):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np
    b, H, d = 2, 4, 128
    H_q = H * G
    r = gen.rng(98, G, 0, 0)
    q = gen.to_storage(r.standard_normal((b, H_q, d)), dtype)
    fR = r.standard_normal((b, H_q, d)).astype(np.float32)
    lse = (r.standard_normal((b, H_q)) * 3 + 5).astype(np.float32)
    moms = _moments(b, H, d, 40, seed=G)
    moms[1][2] = mk.empty(d)   # a head with nothing evicted
    got = to_np(api.kvm_moment_readout(to_dev(q), to_dev(fR), to_dev(lse), _dev_moments(moms)))
    qd = gen.from_storage(q, dtype)
    for i in range(b):
        for h in range(H_q):
            m32 = {k: (np.float32(v).astype(np.float64) if k != "n" else v) for k, v in moms[i][h // G].items()}
            ref, _ = mk.mix(qd[i, h], fR[i, h].astype(np.float64), float(lse[i, h]), m32, d)
            np.testing.assert_allclose(got[i, h], ref, rtol=1e-5, atol=1e-5 * np.abs(ref).max())


@pytest.mark.parametrize("L,B,b,T", [(2048, 128, 1, 6), (1500, 200, 2, 4)])
def test_momentkv_prefill_and_decode(L, B, b, T):
    """The whole moment-informed prefill and the decode with the NC mix, every (sequence, KV
    head) pair compared until a near-tie (the 1e-5 rule); most pairs must go through every
    round and the decode."""
    from learned_kv_cache_mqa_amd import api
    from tests.flows import momentkv_compare
    cfg = WORKLOADS["qwen3_4b_momentkv_32k"].with_(L=L, B=B, b=b, T=T)
    p = gen.make_prefill(cfg)
    dec = gen.make_decode(cfg, steps=T)
    pairs = [(i, g) for i in range(b) for g in range(cfg.H_kv)]
    n_dec, n_rounds = momentkv_compare(p, pairs, B, T, dec, api.cache_cap(B + T))
    assert n_dec >= len(pairs) // 2, f"only {n_dec} of {len(pairs)} pairs reached the decode"
