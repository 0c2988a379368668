"""Shared helpers for the GPU parity tests (oracle comparisons)."""
import numpy as np
import torch

from workloads import to_f64_numpy

# Bar for a floating-point output: normwise maximum relative error
# max|gpu - oracle| / max|oracle| per output tensor.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def rel_err(gpu, ref):
    g = gpu.detach().to("cpu", torch.float64).numpy() if torch.is_tensor(gpu) else np.asarray(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    if not np.all(np.isfinite(g)):
        return float("inf")
    return float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-30))


def assert_close(name, gpu, ref, dtype, tol=None):
    e = rel_err(gpu, ref)
    bar = TOL[dtype] if tol is None else tol
    print(f"  {name}: max-rel {e:.3e} (bar {bar:.0e})", flush=True)
    assert e <= bar, f"{name}: max-rel error {e:.3e} > {bar:.0e}"
    return e


def f64(inp, names=None):
    return {n: to_f64_numpy(t) for n, t in inp.items() if names is None or n in names}


def to_dev(inp):
    return {n: t.cuda() for n, t in inp.items()}
