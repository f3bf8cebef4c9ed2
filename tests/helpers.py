"""Shared helpers of the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

# Pass bar for fp32-state outputs and checkpoints, per element, relative to
# the fp64 oracle: |gpu - oracle| <= RTOL * max(1, |oracle|).
RTOL = 2e-5


def rel_err(gpu, ref) -> float:
    g = gpu.detach().double().cpu().numpy() if hasattr(gpu, "detach") else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    return float((np.abs(g - r) / np.maximum(1.0, np.abs(r))).max())


def assert_close(gpu, ref, what: str, rtol: float = RTOL):
    e = rel_err(gpu, ref)
    assert np.isfinite(e) and e <= rtol, f"{what}: max scaled error {e:.3e} > {rtol:.1e}"


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
