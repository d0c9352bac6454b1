"""Shared test helpers: error metric, tolerances, oracle inputs in float64."""

import numpy as np

# Normwise relative error of one tensor: max|gpu - ref| / max|ref| (elementwise
# ratios explode near zero).  Tolerances: bf16 storage 2e-2, float32 1e-4.
TOL = {"bf16": 2e-2, "f32": 1e-4}


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / den)


def to_np(t):
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def assert_close(name, got, ref, tol):
    e = rel_err(got, ref)
    print(f"  {name}: rel_err={e:.3e} (tol {tol:.0e})", flush=True)
    assert e <= tol, f"{name}: normwise relative error {e:.3e} > {tol:.0e}"
    return e


def oracle_pack(samples):
    from oracle import pack as P

    return P.pack(samples)


def f64_block(nb):
    return {s: {k: np.asarray(v, np.float64) for k, v in nb[s].items()} for s in nb}
