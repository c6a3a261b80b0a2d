"""Helpers shared by the GPU parity tests: device upload of the generator's
arrays and the tolerance checks (fp32: 1e-5, bf16 with fp32 accumulation:
2e-3 on the loss and 1e-2 x max|g| on gradients)."""

import os
import sys

import numpy as np
import pytest

# fp16 (10 stored mantissa bits against bf16's 7) is held to the bf16 bar.
TOL = {"f32": {"loss": 1e-5, "grad": 1e-5}, "bf16": {"loss": 2e-3, "grad": 1e-2},
       "f16": {"loss": 2e-3, "grad": 1e-2}}


def torch_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(arr, dtype):
    import torch
    if arr is None:
        return None
    if dtype == "bf16" and arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    if dtype == "f16" and arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.float16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def to_host(t, f64=True):
    """Host copy of a device tensor (bf16 -> exact float values); float64
    unless f64 is False (then float32, for very large gradients)."""
    import torch
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
        a = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    elif t.dtype == torch.float16:
        a = t.detach().cpu().numpy().astype(np.float32)
    else:
        a = t.detach().cpu().numpy()
    return a.astype(np.float64) if f64 else a


def check_scalar(gpu, ref, rtol, what="loss"):
    gpu = float(np.asarray(gpu).reshape(-1)[0])
    if ref == 0.0:
        assert gpu == 0.0, f"{what}: expected exact 0, got {gpu}"
        return
    rel = abs(gpu - ref) / abs(ref)
    assert rel <= rtol, f"{what}: rel err {rel:.3e} > {rtol:.1e} (gpu {gpu!r}, ref {ref!r})"


def check_max_rel(gpu, ref, frac, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    scale = float(np.abs(ref).max())
    err = float(np.abs(gpu - ref).max())
    if scale == 0.0:
        assert err == 0.0, f"{what}: expected exact zeros, max |gpu| {err}"
        return
    assert err <= frac * scale, f"{what}: max err {err:.3e} > {frac:.1e} x max|ref| {scale:.3e}"


def oracle_inputs(inp):
    """float64 views of the exact values the GPU receives."""
    f = lambda a: None if a is None else np.asarray(a, dtype=np.float64)
    return f(inp["X_f32"]), f(inp["W_f32"]), f(inp["bias_f32"]), inp["targets"]


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
