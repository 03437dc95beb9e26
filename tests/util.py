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


# Per-row bound: every row's error must stay within ROW_FACTOR times the
# tolerance of the larger of that row's own norm and the typical (RMS) row
# norm of the reference.  A single wrong row, which the whole-tensor norm
# would dilute, fails it; a row that is small by cancellation is judged
# against the typical row instead of its own tiny norm.
ROW_FACTOR = 5.0


def row_ratio(got, ref):
    """(worst per-row error ratio, its row index) as bounded above."""
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if r.size == 0:
        return 0.0, -1
    n = r.shape[0] if r.ndim >= 1 else 1
    g2, r2 = g.reshape(n, -1), r.reshape(n, -1)
    typ = np.linalg.norm(r2) / np.sqrt(n)
    den = np.maximum(np.linalg.norm(r2, axis=1), typ)
    err = np.linalg.norm(g2 - r2, axis=1)
    ratio = np.where(den > 0, err / np.where(den > 0, den, 1.0), err)
    i = int(np.argmax(ratio))
    return float(ratio[i]), i


def assert_close(name, got, ref, dtype, factor=1.0):
    e = rel_fro(got, ref)
    tol = TOL[dtype] * factor
    rr, ri = row_ratio(got, ref)
    print(f"  {name}: rel_fro={e:.3e} max_abs={max_abs(got, ref):.3e} worst_row={rr:.3e}@{ri} (tol {tol:.0e}, "
          f"row {ROW_FACTOR * tol:.0e})", flush=True)
    assert e <= tol, f"{name}: relative Frobenius error {e:.3e} > {tol:.0e}"
    assert rr <= ROW_FACTOR * tol, f"{name}: row {ri} relative error {rr:.3e} > {ROW_FACTOR * tol:.0e}"
