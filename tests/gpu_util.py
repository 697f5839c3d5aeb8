"""Helpers for the GPU parity tests: move seeded inputs to the GPU and compare
GPU results with the oracle element by element."""
from __future__ import annotations

import numpy as np

# Tolerances: bf16 storage with fp32 accumulation, and the fp32 path.
TOL_BF16_O = 2e-2
TOL_BF16_LSE = 1e-3
TOL_F32 = 1e-4


def to_gpu(arr_store: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr_store).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr_store, dtype=np.float32))
    return t.to("cuda", non_blocking=False)


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def report(name, o_gpu, o_ref, lse_gpu=None, lse_ref=None):
    do = np.abs(o_gpu - o_ref)
    msg = f"{name}: max|dO|={do.max():.3e} relRMS={np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-300):.3e}"
    if lse_gpu is not None:
        msg += f" max|dLSE|={np.abs(lse_gpu - lse_ref).max():.3e}"
    print(msg, flush=True)
    return msg


def assert_close(o_gpu, o_ref, lse_gpu=None, lse_ref=None, *, dtype="bf16", name=""):
    tol_o = TOL_BF16_O if dtype == "bf16" else TOL_F32
    tol_l = TOL_BF16_LSE if dtype == "bf16" else TOL_F32
    assert np.all(np.isfinite(o_gpu)), f"{name}: non-finite output"
    msg = report(name, o_gpu, o_ref, lse_gpu, lse_ref)
    assert np.abs(o_gpu - o_ref).max() <= tol_o, msg
    if lse_gpu is not None:
        assert np.all(np.isfinite(lse_gpu)), f"{name}: non-finite LSE"
        assert np.abs(lse_gpu - lse_ref).max() <= tol_l, msg
