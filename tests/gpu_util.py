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
