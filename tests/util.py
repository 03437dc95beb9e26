"""Helpers shared by the tests (no arithmetic of the module here)."""
import numpy as np
import torch

TOL = {"f32": 1e-5, "bf16": 2e-2}


def rel_fro(got, ref):
    """Relative Frobenius error ||got - ref|| / ||ref|| (fp64)."""
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / den) if den > 0 else float(np.linalg.norm(g - r))


def max_abs(got, ref):
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    return float(np.max(np.abs(g - np.asarray(ref, np.float64)))) if g.size else 0.0


def tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(x, dtype, dev):
    """float32 numpy (already rounded to `dtype`) -> device tensor of `dtype` (exact)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(tdt(dtype))


def f32_dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def i64_dev(x, dev):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int64)).to(dev)


def host(t):
    return t.detach().double().cpu().numpy()


def assert_close(name, got, ref, dtype, factor=1.0):
    e = rel_fro(got, ref)
    tol = TOL[dtype] * factor
    print(f"  {name}: rel_fro={e:.3e} max_abs={max_abs(got, ref):.3e} (tol {tol:.0e})", flush=True)
    assert e <= tol, f"{name}: relative Frobenius error {e:.3e} > {tol:.0e}"
