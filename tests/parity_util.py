"""Comparison helpers for GPU-vs-oracle parity (tolerances of the mixer's spec).

fp32 inputs: relative L2 <= 1e-5.  bf16 inputs (fp32 state and accumulation):
relative L2 <= 1e-2 and max |x - ref| <= 5e-2 * max |ref|.  Checked per tensor
and per sequence (every batch entry against its own reference).
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": (1e-5, None), "bf16": (1e-2, 5e-2)}


def f64(t):
    return t.detach().double().cpu().numpy()


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(got - ref) / (nref if nref > 0 else 1.0)
    mref = np.abs(ref).max() if ref.size else 0.0
    mx = (np.abs(got - ref).max() / (mref if mref > 0 else 1.0)) if ref.size else 0.0
    return rel, mx


def assert_close(got, ref, dtype, name, batch_axis=0):
    rel_tol, max_tol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    rel, mx = errors(got, ref)
    assert rel <= rel_tol, f"{name}: rel L2 {rel:.3e} > {rel_tol}"
    if max_tol is not None:
        assert mx <= max_tol, f"{name}: max err {mx:.3e} > {max_tol} * max|ref|"
    if batch_axis is not None and got.ndim > 1 and got.shape[batch_axis] > 1:
        for b in range(got.shape[batch_axis]):
            gb = np.take(got, b, axis=batch_axis)
            rb = np.take(ref, b, axis=batch_axis)
            r2, m2 = errors(gb, rb)
            assert r2 <= rel_tol, f"{name}[{b}]: rel L2 {r2:.3e} > {rel_tol}"
            if max_tol is not None:
                assert m2 <= max_tol, f"{name}[{b}]: max err {m2:.3e}"
    return rel, mx


def assert_close_groups(got, ref, groups, dtype, name):
    """A per-head vector (dlambda) checked as a whole and on each group of heads on its
    own (e.g. the lambda = 0, lambda = 1 and interior heads), so that components of a
    small group are not hidden behind the large ones of another."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert_close(got, ref, dtype, name, batch_axis=None)
    for label, idx in groups.items():
        if len(idx):
            assert_close(got[list(idx)], ref[list(idx)], dtype, f"{name}[{label}]", batch_axis=None)


def lambda_groups(lams):
    """Head indices with lambda == 0, lambda == 1 and the rest."""
    lams = [float(x) for x in lams]
    return {"zero": [h for h, x in enumerate(lams) if x == 0.0],
            "one": [h for h, x in enumerate(lams) if x == 1.0],
            "interior": [h for h, x in enumerate(lams) if 0.0 < x < 1.0]}
