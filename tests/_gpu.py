"""Helpers for the GPU parity tests: move seeded inputs to the device, read results back as
float64, and compare with the oracle using the tolerance metric
err = max|a - r| / max(max|r|, 1e-30) per tensor."""
import numpy as np
import torch

DEV = "cuda:0"
# fp16 (not stated by the pages): the bf16 bound scaled by the ratio of the unit
# roundoffs, 2^-11 / 2^-8 = 1/8, since every rounding point is the same and only the format
# changes
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2.5e-3}
_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def dev(arr, dtype):
    """numpy fp32 (exactly representable in dtype) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(arr, np.float32))
    t = t.to(_TORCH[dtype])
    return t.to(DEV)


def empty(shape, dtype):
    return torch.empty(shape, dtype=_TORCH[dtype],
                       device=DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(a, r, scale=None):
    """max|a - r| / max|r|; `scale` replaces max|r| for a reference that is identically zero
    (then the error is measured against the size of a sibling output of the same op)."""
    a = np.asarray(a, np.float64)
    r = np.asarray(r, np.float64)
    assert a.shape == r.shape, (a.shape, r.shape)
    assert np.all(np.isfinite(a)), "non-finite values in the GPU result"
    den = float(np.max(np.abs(r))) if r.size else 0.0
    if den == 0.0 and scale is not None:
        den = scale
    return float(np.max(np.abs(a - r)) / max(den, 1e-30)) if a.size else 0.0


def assert_close(a, r, dtype, what, tol=None, scale=None):
    e = rel_err(a, r, scale)
    lim = TOL[dtype] if tol is None else tol
    print(f"  {what}: rel err {e:.3e} (limit {lim:.1e})", flush=True)
    assert e <= lim, f"{what}: rel err {e:.3e} > {lim:.1e}"


def ws(nbytes):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


def stream():
    return torch.cuda.current_stream()
