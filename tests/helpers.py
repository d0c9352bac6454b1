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


# Row-wise form of the same metric: max over rows r of max|gpu_r - ref_r| /
# max(max|ref_r|, ROW_FLOOR * max|ref|).  A wrong small-magnitude row (a
# text row beside large image rows, one weight-gradient row) fails it even
# when the tensor's largest row sets the normwise scale; rows far below the
# tensor's scale are judged against ROW_FLOOR of it, where bf16 rounding of
# the shared operands, not the row's own size, sets the error.
ROW_FLOOR = 1e-2
# Row-wise bound of the bfloat16 weight gradients: a row of dW is a sum over
# tokens whose terms cancel (per-sample adaLN rows most), so its relative
# error is the unit roundoff times the row's condition number, not the
# unit roundoff; 0.25 still fails a row that is wrong (off by O(1)).
ROW_TOL_WGRAD_BF16 = 0.25


def rel_err_rows(got, ref, floor=ROW_FLOOR):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    # a vector is one row
    g2 = got.reshape(got.shape[0], -1) if got.ndim > 1 else got.reshape(1, -1)
    r2 = ref.reshape(ref.shape[0], -1) if ref.ndim > 1 else ref.reshape(1, -1)
    top = np.max(np.abs(r2))
    if top == 0:
        return float(np.max(np.abs(g2)))
    den = np.maximum(np.max(np.abs(r2), axis=1), floor * top)
    return float(np.max(np.max(np.abs(g2 - r2), axis=1) / den))


def to_np(t):
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def assert_close(name, got, ref, tol, rows=False):
    """Normwise check at tol; rows=True adds the row-wise check at tol, a
    number gives the row-wise check its own bound."""
    e = rel_err(got, ref)
    er = rel_err_rows(got, ref) if rows is not False else None
    rtol = tol if rows is True else rows
    extra = f", row-wise {er:.3e} (bound {rtol:.3g})" if er is not None else ""
    print(f"  {name}: rel_err={e:.3e} (bound {tol:.3g}: {e / tol:.0%} of it){extra}", flush=True)
    assert e <= tol, f"{name}: normwise relative error {e:.3e} > {tol:.3g}"
    if er is not None:
        assert er <= rtol, f"{name}: row-wise relative error {er:.3e} > {rtol:.3g}"
    return e


def oracle_pack(samples):
    from oracle import pack as P

    return P.pack(samples)


def f64_block(nb):
    return {s: {k: np.asarray(v, np.float64) for k, v in nb[s].items()} for s in nb}
