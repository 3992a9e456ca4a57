"""Shared helpers of the GPU parity tests: upload stored inputs, compare
against the oracle with the normwise relative error."""
import numpy as np
import torch

import workloads as wl
from workloads.device import dev  # noqa: F401  (re-exported for the tests)

TOL = {wl.DT_F32: 1e-4, wl.DT_BF16: 2e-2}


def host_f64(t):
    """GPU tensor -> float64 numpy (exact decode of bf16/fp32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def rowwise_err(got, ref):
    """max over rows of max|got - ref| / max|ref| (one row = last axis)."""
    got = np.asarray(got, np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((np.abs(got - ref).max(axis=1) / den).max())
