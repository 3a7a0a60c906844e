"""kvm_decode_attn_mem_noalloc (split states in the library's own per-device scratch array,
for callers that cannot allocate) against kvm_decode_attn_mem with a caller workspace:
the same kernels, so the outputs must be bitwise identical, on two calls in a row, the
second with a smaller input; plus the oracle bar on the first."""
import math

import numpy as np
import pytest

from oracle import indexmem as im
from synth import gen

pytestmark = pytest.mark.gpu


def _inputs(r, b, H_q, H_kv, d, cap):
    st = lambda x: gen.to_storage(x, "bf16")
    M = np.zeros((b, H_kv, d, d))
    bv = np.zeros((b, H_kv, d))
    for i in range(b):
        for g in range(H_kv):
            M[i, g], bv[i, g] = im.memory_build(r.standard_normal((20, d)), r.standard_normal((20, d)), 0.99)
    return dict(Kc=st(r.standard_normal((b, H_kv, cap, d))), Vc=st(r.standard_normal((b, H_kv, cap, d))),
                q=st(r.standard_normal((b, H_q, d))), kn=st(r.standard_normal((b, H_kv, d))),
                vn=st(r.standard_normal((b, H_kv, d))), w_g=st(r.standard_normal((H_q, d)) / math.sqrt(d)),
                M=M.astype(np.float32), bv=bv.astype(np.float32))


def _run(c, lens, noalloc):
    import torch
    from learned_kv_cache_mqa_amd import api
    from tests.gpu_util import to_dev, to_np
    Kc, Vc = to_dev(c["Kc"]), to_dev(np.ascontiguousarray(c["Vc"].transpose(0, 1, 3, 2)))
    b, H_q = c["q"].shape[:2]
    o = torch.empty((b, H_q, c["q"].shape[2]), dtype=torch.float32, device=Kc.device)
    lse = torch.empty((b, H_q), dtype=torch.float32, device=Kc.device)
    fn = api.kvm_decode_attn_mem_noalloc if noalloc else api.kvm_decode_attn_mem
    fn(to_dev(c["q"]), Kc, Vc, to_dev(np.array(lens, np.int32)), k_new=to_dev(c["kn"]), v_new=to_dev(c["vn"]),
       M=to_dev(c["M"]), bvec=to_dev(c["bv"]), w_g=to_dev(c["w_g"]), o=o, lse=lse)
    torch.cuda.synchronize()
    return to_np(o), to_np(lse), to_np(Kc), to_np(Vc)


def test_noalloc_decode_matches_workspace_decode():
    r = gen.rng(97, 1, 0, 0)
    # the 16K workload's decode shape, then a smaller one (fewer sequences, shorter caches),
    # then a mid-sized one (more splits per pair than the first)
    shapes = [(8, 32, 8, 128, 2176, [1894 - 7 * i for i in range(8)]), (2, 32, 8, 128, 704, [410, 333]),
              (4, 32, 8, 128, 2176, [1894 - 7 * i for i in range(4)])]
    for n, (b, H_q, H_kv, d, cap, lens) in enumerate(shapes):
        c = _inputs(r, b, H_q, H_kv, d, cap)
        got = _run(c, lens, True)
        want = _run(c, lens, False)
        for x, y, what in zip(got, want, ("o", "lse", "Kc", "Vc")):
            assert x.tobytes() == y.tobytes(), f"call {n}: {what} differs from the workspace entry point"
        if n == 0:
            f = lambda x: gen.from_storage(x, "bf16")
            for i in (0, b - 1):
                K, V = f(c["Kc"][i]).copy(), f(c["Vc"][i]).copy()
                K[:, lens[i]], V[:, lens[i]] = f(c["kn"][i]), f(c["vn"][i])
                ref, _ = im.decode_attention(f(c["q"][i]), K, V, lens[i] + 1, 1 / math.sqrt(d))
                m, g = im.memory_readout(f(c["q"][i]), c["M"][i].astype(np.float64), c["bv"][i].astype(np.float64),
                                         f(c["w_g"]), 1e-6)
                ref = im.residual_output(ref, m, g)
                np.testing.assert_allclose(got[0][i], ref, rtol=2e-4, atol=2e-4 * np.abs(ref).max())
