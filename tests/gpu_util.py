"""Helpers shared by the GPU parity tests: moving seeded storage-format inputs to the
device and the comparison rules."""
import numpy as np
import pytest
import torch

from synth import gen


def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU test started without a visible GPU")
    return torch.device("cuda", 0)


def to_dev(a, dtype=None):
    """Storage-format numpy array -> device tensor (uint16 -> bfloat16 bit-exact)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    if a.dtype == np.float64:
        a = a.astype(np.float32 if dtype is None else dtype)
    return torch.from_numpy(a).to(dev())


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def decode_store(a, dtype):
    """Storage -> float64 (exact)."""
    return gen.from_storage(a, dtype)


def normwise(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def maxabs(got, ref):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))


def assert_output(got, ref, dtype, what=""):
    """The output bar: max-abs 1e-4 for fp32 workloads, normwise relative 2e-2 for bf16."""
    if dtype == "f32":
        e = maxabs(got, ref)
        assert e <= 1e-4, f"{what}: max-abs error {e:.3e} > 1e-4"
    else:
        e = normwise(got, ref)
        assert e <= 2e-2, f"{what}: normwise error {e:.3e} > 2e-2"
    return e


def set_check(gpu_kept, I_ref, B, R, inclusive=True, rel=1e-5):
    """Index-set rule: the GPU's kept set must equal the oracle's outside the band of
    scores within `rel` of the oracle's n_top-th selected score, and have the same size.
    The oracle takes the decision on its scores rounded to fp32 (the kernel's precision).
    Returns the number of positions inside the band where the two sets differ."""
    from oracle import indexmem as im
    I32 = np.asarray(I_ref, np.float64).astype(np.float32).astype(np.float64)
    L = len(I32)
    ref_idx, _ = im.topk_select(I32, B, R, inclusive)
    g = set(int(x) for x in np.asarray(gpu_kept).tolist())
    r = set(ref_idx.tolist())
    assert len(g) == len(r), f"kept {len(g)} != {len(r)}"
    n_cand = L - min(R, L)
    n_top = B - R if inclusive else B
    if n_top >= n_cand or n_top <= 0:
        assert g == r
        return 0
    cand_sel = [t for t in ref_idx.tolist() if t < n_cand]
    tau = min(I32[t] for t in cand_sel)
    band = np.abs(I32 - tau) <= rel * abs(tau)
    diff = g ^ r
    bad = [t for t in diff if not band[t]]
    assert not bad, f"set mismatch outside the 1e-5 band at {bad[:10]} (tau={tau})"
    return len(diff)
