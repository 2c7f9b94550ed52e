"""Helpers shared by the GPU parity tests (no method arithmetic here)."""
import numpy as np
import pytest
import torch

F32_TOL = 1e-4     # float32 results: normwise max |gpu - ref| / max |ref|
LOSS_TOL = 1e-5    # loss: |gpu - ref| / |ref|
BF16_TOL = 2e-2    # bf16-operand / float32-accumulate results
F16_TOL = 5e-3     # half-operand / float32-accumulate results (about 10 half ulps)


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a HIP device")
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(device())
    return t if dtype is None else t.to(dtype)


def to_np(t):
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def normwise(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    assert a.shape == ref.shape, (a.shape, ref.shape)
    d = np.max(np.abs(ref)) if ref.size else 0.0
    e = np.max(np.abs(a - ref)) if ref.size else 0.0
    return float(e / d) if d > 0 else float(e)


def assert_close(a, ref, tol, what=""):
    err = normwise(a, ref)
    assert err < tol, f"{what}: normwise error {err:.3e} >= {tol:.1e}"
    return err


def misaligned(t: torch.Tensor) -> torch.Tensor:
    """Same values, data pointer 4 bytes past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = flat[1:].view(t.shape)
    v.copy_(t)
    return v
