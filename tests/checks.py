"""Comparisons of the HIP path's values with the oracle's (no GPU needed here).

Three checks, each with its own bound:

* ``out`` (bf16 or fp32 storage): element by element within ``atol + rtol*|ref|``
  (bf16: the 1e-2 absolute / 2e-2 relative bound stated for the method's bf16
  outputs accumulated in fp32), and row by row (a row is one (token, head)
  vector of head_dim values): ``max|got - ref| <= rtol * max|ref|``.  The row
  check keeps its meaning where the values themselves are small: at a 64K
  prefix a dense row's elements have a spread of about 0.006, below the
  elementwise absolute bound.
* ``o_p`` cache rows (fp32): the same two checks.
* ``L_p`` cache (fp32, natural log): absolute error in nats.  With bf16
  inputs the softmax weights fed to the PV product are rounded to bf16, and
  the row sum is taken over the rounded weights; a sum of weights each off by
  at most 2^-9 relative is off by at most 2^-9 relative, i.e. 1.95e-3 nats in
  L_p, plus fp32 accumulation (1e-6 relative per term, far smaller).  The
  bound is twice that: 4e-3 nats.  Dropping one page of a ~100-page union
  moves L_p by about ln(1 - 1/100) = -0.01 nats, well outside it.
  With fp32 inputs nothing is rounded to bf16: 1e-4 nats.

Every comparison returns a short record of its errors, which the GPU tests
print, so that a run shows how much margin each bound keeps.
"""
from __future__ import annotations

import numpy as np

TOL = {"bf16": dict(rtol=2e-2, atol=1e-2), "f32": dict(rtol=1e-4, atol=1e-5)}
LP_ATOL = {"bf16": 4e-3, "f32": 1e-4}


def _finite_pair(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    return np.where(both_inf, 0.0, got), np.where(both_inf, 0.0, ref)


def value_errors(got, ref, dtype):
    """Elementwise and per-row (last axis) errors of a value array."""
    g, r = _finite_pair(got, ref)
    tol = TOL[dtype]
    d = np.abs(g - r)
    bad_el = ~(d <= tol["atol"] + tol["rtol"] * np.abs(r))
    row_err = d.max(axis=-1) if d.ndim else d
    row_ref = np.abs(r).max(axis=-1) if r.ndim else np.abs(r)
    bad_row = ~(row_err <= tol["rtol"] * row_ref)
    # rows whose reference is exactly zero (empty prefix) must match exactly
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(row_ref > 0, row_err / np.where(row_ref > 0, row_ref, 1.0),
                       np.where(row_err > 0, np.inf, 0.0))
    return dict(max_abs=float(d.max()) if d.size else 0.0,
                max_row_rel=float(rel.max()) if rel.size else 0.0,
                n_bad_el=int(bad_el.sum()), n_bad_row=int(bad_row.sum()),
                first_bad_el=np.argwhere(bad_el)[:3].tolist(),
                first_bad_row=np.argwhere(bad_row)[:3].tolist(), size=int(d.size))


def lp_errors(got, ref, dtype):
    g, r = _finite_pair(got, ref)
    d = np.abs(g - r)
    bad = ~(d <= LP_ATOL[dtype])  # also catches a -inf on one side only (nan/inf distance)
    return dict(max_abs=float(np.nanmax(d)) if d.size else 0.0, n_bad=int(bad.sum()),
                first_bad=np.argwhere(bad)[:3].tolist(), size=int(d.size))


def check_values(got, ref, dtype, what):
    e = value_errors(got, ref, dtype)
    if e["n_bad_el"] or e["n_bad_row"]:
        raise AssertionError(
            f"{what}: {e['n_bad_el']} of {e['size']} elements and {e['n_bad_row']} rows outside "
            f"tolerance (first elements {e['first_bad_el']}, rows {e['first_bad_row']}); "
            f"max abs err {e['max_abs']:.3g}, max row-relative err {e['max_row_rel']:.3g}")
    return f"{what}: max abs {e['max_abs']:.2e}, max row-rel {e['max_row_rel']:.2e}"


def check_lp(got, ref, dtype, what):
    e = lp_errors(got, ref, dtype)
    if e["n_bad"]:
        raise AssertionError(f"{what}: {e['n_bad']} of {e['size']} log-normalisers off by more "
                             f"than {LP_ATOL[dtype]} nats (first {e['first_bad']}); max abs err "
                             f"{e['max_abs']:.3g}")
    return f"{what}: max abs {e['max_abs']:.2e} nats"
