"""Helpers for the GPU tests: device selection and the parity metric.

The parity metric is max-abs error relative to the reference's largest
magnitude, in float64: err(X) = max|X_gpu - X_ref| / max|X_ref| (absolute
error when the reference is all zero).
"""
import os

import numpy as np
import pytest
import torch

TOL_O = 1e-4        # forward output
TOL_LSE = 1e-4      # forward log-sum-exp
TOL_GRAD = 1e-3     # dQ, dK, dV
TOL_DECODE = 1e-5   # paged decode vs dense decode on the gathered KV


def require_gpu():
    if not torch.cuda.is_available():
        if os.environ.get("ATTN_REQUIRE_GPU") == "1":
            pytest.fail("ATTN_REQUIRE_GPU=1 but no GPU is visible")
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def rel_err(gpu, ref):
    g = gpu.detach().double().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = ref.detach().double().cpu().numpy() if isinstance(ref, torch.Tensor) else np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    den = float(np.max(np.abs(r)))
    num = float(np.max(np.abs(g - r)))
    return num / den if den > 0 else num


def announce(msg):
    """Name the case on stdout (flushed) before a GPU step."""
    print(f"[gpu-case] {msg}", flush=True)
