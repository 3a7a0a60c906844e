"""The attention-state memory (ASM) on the GPU against the oracle: prefix attention states,
K-means, the per-cluster states, cosine retrieval with the merge, and the whole pipeline.

Synthetic inputs: the prefix K, V ~ N(0, 1); calibration and decode queries from a mixture
of Gaussians per head (centres ~ N(0, 1), spread 0.3), all rounded to bf16."""
import math

import numpy as np
import pytest

from oracle import asm
from oracle import indexmem as im
from synth import gen

pytestmark = pytest.mark.gpu

BF = "bf16"


def _bf(x):
    return gen.to_storage(x, BF)


def _f(x):
    return gen.from_storage(x, BF)


def _seeds(X, lab, K, nc):
    """Initial centroids [H, K, d] f32: one query of each true centre, then far-away points
    that draw no member (they must stay where they are)."""
    H, d = X.shape[1], X.shape[2]
    C0 = np.zeros((H, K, d))
    for h in range(H):
        for k in range(K):
            C0[h, k] = X[int(np.argmax(lab[h] == k)), h] if k < nc else 50.0 + k
    return C0.astype(np.float32)


def _mixture(r, n, H, d, n_centres, spread=0.3):
    """n queries per head around n_centres centres per head: [n, H, d], plus the labels."""
    centres = r.standard_normal((H, n_centres, d))
    lab = r.integers(0, n_centres, size=(H, n))
    X = np.stack([centres[h, lab[h]] + spread * r.standard_normal((n, d)) for h in range(H)], axis=1)
    return X, lab


PREFIX_CASES = [
    # N, H_q, H_kv, d, L, head-major prefix
    (100, 8, 2, 128, 300, False),
    (64, 4, 4, 64, 1000, True),
    (33, 32, 8, 128, 257, False),
    (40, 16, 2, 64, 95, False),
]


@pytest.mark.parametrize("N,H_q,H_kv,d,L,hm", PREFIX_CASES)
def test_prefix_states_match_oracle(N, H_q, H_kv, d, L, hm):
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np
    r = gen.rng(200, N, L, d)
    Q = _bf(r.standard_normal((N, H_q, d)))
    K = _bf(r.standard_normal((L, H_kv, d)))
    V = _bf(r.standard_normal((L, H_kv, d)))
    tr = (lambda x: np.ascontiguousarray(x.transpose(1, 0, 2))) if hm else (lambda x: x)
    a, lse = api.kvm_asm_prefix_states(to_dev(Q), to_dev(tr(K)), to_dev(tr(V)), kv_head_major=hm)
    a, lse = to_np(a), to_np(lse)
    ra, rl = asm.prefix_states(_f(Q), _f(K), _f(V), 1 / math.sqrt(d))
    # P enters the matrix cores as bf16 hi + lo (16 bits), fp32 accumulation
    np.testing.assert_allclose(a, ra, rtol=2e-4, atol=2e-4 * np.abs(ra).max())
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-4 * np.abs(rl).max())


def test_prefix_states_in_chunks_match_oracle():
    """A prefix encoded in three uneven chunks, each merged into the states of the earlier
    ones, against the oracle's states over the whole prefix."""
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np
    r = gen.rng(205, 0, 0, 0)
    N, H_q, H_kv, d, cuts = 70, 8, 2, 128, [0, 130, 131, 500]
    Q = _bf(r.standard_normal((N, H_q, d)))
    K = _bf(r.standard_normal((cuts[-1], H_kv, d)))
    V = _bf(r.standard_normal((cuts[-1], H_kv, d)))
    a = lse = None
    for c0, c1 in zip(cuts, cuts[1:]):
        a, lse = api.kvm_asm_prefix_states(to_dev(Q), to_dev(np.ascontiguousarray(K[c0:c1])),
                                           to_dev(np.ascontiguousarray(V[c0:c1])), a=a, lse=lse,
                                           accumulate=c0 > 0)
    ra, rl = asm.prefix_states(_f(Q), _f(K), _f(V), 1 / math.sqrt(d))
    np.testing.assert_allclose(to_np(a), ra, rtol=2e-4, atol=2e-4 * np.abs(ra).max())
    np.testing.assert_allclose(to_np(lse), rl, rtol=0, atol=1e-4 * np.abs(rl).max())


KMEANS_CASES = [
    # N, H, d, K, iters, true centres
    (600, 4, 128, 16, 5, 16),
    (1100, 2, 64, 24, 3, 20),     # more than two 512-row chunks, 4 centroids drawing nobody
    (70, 3, 128, 8, 0, 8),        # assignment only
    # several 32-centroid tiles through the assignment's three-slot ring: 3 tiles (the loop
    # without a tail), 4 (one tail step), 2 (two tail steps)
    (900, 2, 128, 96, 2, 96),
    (700, 2, 64, 100, 2, 100),
    (500, 3, 128, 40, 2, 40),
]


@pytest.mark.parametrize("N,H,d,K,iters,nc", KMEANS_CASES)
def test_kmeans_matches_oracle(N, H, d, K, iters, nc):
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np
    r = gen.rng(201, N, K, d)
    Xm, lab = _mixture(r, N, H, d, nc)
    Xs = _bf(Xm)
    X = _f(Xs)
    C0 = _seeds(X, lab, K, nc)
    Cd = to_dev(C0)
    idx = to_np(api.kvm_asm_kmeans(to_dev(Xs), Cd, iters))
    Cg = to_np(Cd)
    for h in range(H):
        Cr, ir = asm.kmeans(X[:, h], C0[h].astype(np.float64), iters)
        # one seed per separated cluster: no assignment lies near a tie (checked), so the
        # assignments must agree exactly
        _, d2 = asm.kmeans_assign(X[:, h], Cr)
        s = np.sort(d2, axis=1)
        assert (s[:, 1] - s[:, 0] > 1e-3 * s[:, 1]).all()
        np.testing.assert_array_equal(idx[h], ir)
        np.testing.assert_allclose(Cg[h], Cr, rtol=1e-5, atol=1e-6)


def _d2(X, C):
    """Squared distances [N, K] in fp64 (for validity checks of the GPU's own results)."""
    return (X * X).sum(1)[:, None] - 2.0 * X @ C.T + (C * C).sum(1)[None, :]


def test_kmeans_benchmark_seeding_band():
    """K-means as the benchmark seeds it: unclustered N(0, 1) queries, the first K queries as
    the initial centroids, so near-ties between centroids do occur.  Per head and iteration t
    (the library run for t rounds), the assignment must equal the oracle's except at points
    whose two candidate distances agree to 1e-5 (after such a point the trajectories
    legitimately part, and that head is no longer compared with the oracle); the centroids
    must match while the assignments agree.  At every t the GPU's own trajectory must also be
    valid: each point at a nearest centroid of C_t (within the band), and C_t the mean of the
    members under the previous assignment (a centroid without members stays)."""
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np
    N, H, d, K, iters = 2048, 2, 128, 128, 6
    r = gen.rng(203, 0, 0, 0)
    Xs = _bf(r.standard_normal((N, H, d)))
    X = _f(Xs)
    C0 = np.ascontiguousarray(X[:K].transpose(1, 0, 2)).astype(np.float32)
    Cs, ids = [], []
    for t in range(iters + 1):
        Cd = to_dev(C0)
        ids.append(to_np(api.kvm_asm_kmeans(to_dev(Xs), Cd, t)))
        Cs.append(to_np(Cd).astype(np.float64))
    compared = 0
    for h in range(H):
        Xh = X[:, h]
        # validity of the GPU's own trajectory
        for t in range(iters + 1):
            d2 = _d2(Xh, Cs[t][h])
            got = d2[np.arange(N), ids[t][h]]
            assert (got <= d2.min(1) * (1 + 1e-5) + 1e-9).all(), f"head {h} t {t}: a point not at a nearest centroid"
            if t:
                for k in range(K):
                    m = ids[t - 1][h] == k
                    want = Xh[m].mean(0) if m.any() else Cs[t - 1][h][k]
                    np.testing.assert_allclose(Cs[t][h][k], want, rtol=1e-5, atol=1e-5)
        # against the oracle's trajectory, until a near-tie
        C = C0[h].astype(np.float64)
        idx_r, d2r = asm.kmeans_assign(Xh, C)
        for t in range(iters + 1):
            if t:
                C = asm.kmeans_update(Xh, idx_r, C)
                idx_r, d2r = asm.kmeans_assign(Xh, C)
            diff = np.nonzero(ids[t][h] != idx_r)[0]
            if len(diff):
                g = ids[t][h][diff]
                gap = np.abs(d2r[diff, g] - d2r[diff, idx_r[diff]])
                assert (gap <= 1e-5 * d2r[diff, idx_r[diff]]).all(), f"head {h} t {t}: assignment outside the band"
                break
            np.testing.assert_allclose(Cs[t][h], C, rtol=1e-5, atol=1e-6)
            compared += 1
    assert compared >= iters, f"only {compared} iterations compared with the oracle"


def test_cluster_states_match_oracle():
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np
    r = gen.rng(202, 0, 0, 0)
    N, H, d, K = 1300, 3, 128, 40
    a = r.standard_normal((N, H, d)).astype(np.float32)
    lse = (r.standard_normal((N, H)) * 4 + 20).astype(np.float32)
    idx = r.integers(0, K - 3, size=(H, N)).astype(np.int32)        # the last 3 clusters stay empty
    ab, lb = api.kvm_asm_cluster_states(to_dev(a), to_dev(lse), to_dev(idx), K)
    ab, lb = to_np(ab), to_np(lb)
    for h in range(H):
        ra, rl = asm.aggregate(a[:, h].astype(np.float64), lse[:, h].astype(np.float64), idx[h], K)
        np.testing.assert_allclose(ab[h], ra, rtol=1e-5, atol=1e-5 * np.abs(ra).max())
        np.testing.assert_allclose(lb[h, :K - 3], rl[:K - 3], rtol=1e-6)
        assert np.isneginf(lb[h, K - 3:]).all() and not ab[h, K - 3:].any()


@pytest.mark.parametrize("b,H,d,K", [(4, 8, 128, 64), (3, 4, 64, 200), (1, 32, 128, 256)])
def test_lookup_merge_matches_oracle(b, H, d, K):
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np
    r = gen.rng(203, b, K, d)
    C = r.standard_normal((H, K, d)).astype(np.float32)
    C *= r.uniform(0.2, 3.0, size=(H, K, 1)).astype(np.float32)     # norms differ: cosine, not dot
    q = _bf(r.standard_normal((b, H, d)))
    ab = r.standard_normal((H, K, d)).astype(np.float32)
    lb = (r.standard_normal((H, K)) * 2 + 5).astype(np.float32)
    ol = r.standard_normal((b, H, d)).astype(np.float32)
    ll = (r.standard_normal((b, H)) * 2 + 5).astype(np.float32)
    o, idx = api.kvm_asm_lookup(to_dev(q), to_dev(C), to_dev(ab), to_dev(lb), to_dev(ol), to_dev(ll))
    o, idx = to_np(o), to_np(idx)
    qd = _f(q)
    for i in range(b):
        for h in range(H):
            k = asm.lookup(qd[i, h], C[h].astype(np.float64))
            if idx[i, h] != k:   # allowed only inside a 1e-6 cosine band
                cos = C[h].astype(np.float64) @ qd[i, h] / np.linalg.norm(C[h], axis=1)
                assert abs(cos[idx[i, h]] - cos[k]) <= 1e-6 * abs(cos[k])
                k = int(idx[i, h])
            ref, _ = im.merge_states([(ol[i, h].astype(np.float64), float(ll[i, h])),
                                      (ab[h, k].astype(np.float64), float(lb[h, k]))])
            np.testing.assert_allclose(o[i, h], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())


def test_asm_pipeline_matches_oracle():
    """Calibration (prefix states, K-means, cluster states) and retrieval for decode
    queries whose local state comes from kvm_decode_attn_mem over the tokens after the
    prefix, against the oracle run end to end from the same inputs."""
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np, assert_output
    r = gen.rng(204, 0, 0, 0)
    N, H_q, H_kv, d, L, Kc, iters, b, Lloc = 400, 8, 2, 128, 700, 12, 4, 3, 40
    centres = r.standard_normal((H_q, Kc, d))
    lab = r.integers(0, Kc, size=(H_q, N + b))
    Xall = np.stack([centres[h, lab[h]] + 0.3 * r.standard_normal((N + b, d)) for h in range(H_q)], axis=1)
    Qs, qs = _bf(Xall[:N]), _bf(Xall[N:])
    Ks, Vs = _bf(r.standard_normal((L, H_kv, d))), _bf(r.standard_normal((L, H_kv, d)))
    Kl, Vl = _bf(r.standard_normal((b, H_kv, Lloc, d))), _bf(r.standard_normal((b, H_kv, Lloc, d)))
    C0 = _seeds(_f(Qs), lab[:, :N], Kc, Kc)

    a, lse = api.kvm_asm_prefix_states(to_dev(Qs), to_dev(Ks), to_dev(Vs))
    Cd = to_dev(C0)
    idx = api.kvm_asm_kmeans(to_dev(Qs), Cd, iters)
    ab, lb = api.kvm_asm_cluster_states(a, lse, idx, Kc)
    cap = api.cache_cap(Lloc)
    Kc_loc = np.zeros((b, H_kv, cap, d), np.uint16)
    Vc_loc = np.zeros((b, H_kv, d, cap), np.uint16)
    Kc_loc[:, :, :Lloc] = Kl
    Vc_loc[:, :, :, :Lloc] = Vl.transpose(0, 1, 3, 2)
    lse_loc = torch.empty((b, H_q), dtype=torch.float32, device="cuda")
    o_loc = api.kvm_decode_attn_mem(to_dev(qs), to_dev(Kc_loc), to_dev(Vc_loc), to_dev(np.full(b, Lloc, np.int32)),
                                    lse=lse_loc)
    o, sel = api.kvm_asm_lookup(to_dev(qs), Cd, ab, lb, o_loc, lse_loc)
    o, sel = to_np(o), to_np(sel)

    sc = 1 / math.sqrt(d)
    ra, rl = asm.prefix_states(_f(Qs), _f(Ks), _f(Vs), sc)
    G = H_q // H_kv
    for h in range(H_q):
        Cr, ir = asm.kmeans(_f(Qs)[:, h], C0[h].astype(np.float64), iters)
        np.testing.assert_array_equal(to_np(idx)[h], ir)
        a_bar, l_bar = asm.aggregate(ra[:, h], rl[:, h], ir, Kc)
        for i in range(b):
            g = h // G
            a_loc, l_loc = im.attention_state(_f(qs)[i, h], _f(Kl)[i, g], _f(Vl)[i, g], sc)
            (ref, _), k = asm.output(_f(qs)[i, h], Cr, a_bar, l_bar, a_loc, l_loc)
            assert sel[i, h] == k
            assert_output(o[i, h], ref, BF, f"query {i} head {h}")
            np.testing.assert_allclose(o[i, h], ref, rtol=2e-4, atol=2e-4 * np.abs(ref).max())
