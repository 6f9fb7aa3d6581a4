"""Helpers for the GPU parity tests: move seeded inputs to the device, read results back as
float64, and compare with the oracle using the tolerance metric
err = max|a - r| / max(max|r|, 1e-30) per tensor."""
import numpy as np
import torch

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def dev(arr, dtype):
    """numpy fp32 (exactly bf16-representable when dtype is bf16) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(arr, np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to(DEV)


def empty(shape, dtype):
    return torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                       device=DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(a, r):
    a = np.asarray(a, np.float64)
    r = np.asarray(r, np.float64)
    assert a.shape == r.shape, (a.shape, r.shape)
    assert np.all(np.isfinite(a)), "non-finite values in the GPU result"
    return float(np.max(np.abs(a - r)) / max(float(np.max(np.abs(r))), 1e-30))


def assert_close(a, r, dtype, what, tol=None):
    e = rel_err(a, r)
    lim = TOL[dtype] if tol is None else tol
    print(f"  {what}: rel err {e:.3e} (limit {lim:.0e})", flush=True)
    assert e <= lim, f"{what}: rel err {e:.3e} > {lim:.0e}"


def ws(nbytes):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


def stream():
    return torch.cuda.current_stream()
