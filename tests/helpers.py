"""Shared helpers for the GPU parity tests: device transfer, the error metric and tolerances.

The parity metric is max|gpu - ref| / max|ref| per output tensor, with ref the fp64 oracle on
the identical (already rounded) inputs.  Bound: 1e-2 for bf16 inputs, 1e-4 for fp32 inputs.
Any non-finite GPU value fails.
"""
import numpy as np

TOL = {"bf16": 1e-2, "f32": 1e-4}


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def dev(x, dtype="f32"):
    """numpy (float32 holding dtype-exact values) -> contiguous cuda tensor of that dtype."""
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device="cuda", dtype=torch_dtype(dtype)).contiguous()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return np.inf
    scale = np.max(np.abs(ref))
    diff = np.max(np.abs(got - ref)) if got.size else 0.0
    return diff / scale if scale > 0 else diff


def assert_close(name, got, ref, dtype):
    e = rel_err(got, ref)
    print(f"  {name}: rel err {e:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert e <= TOL[dtype], f"{name}: max|d|/max|ref| = {e:.3e} > {TOL[dtype]:.0e}"
