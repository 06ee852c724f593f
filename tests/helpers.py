"""Shared test helpers: error metrics and golden-file loading (no scan arithmetic)."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        g = json.load(f)
    ins = {k: (None if v is None else np.asarray(v, dtype=np.float64)) for k, v in g["inputs"].items()}
    return g, ins


def max_rel_err(got, ref, slice_axes=(0, 2)):
    """Max over (b, h) slices of ||got - ref||_inf / ||ref||_inf.

    For y [b,T,H,P] the slice keys are axes (0, 2); for hT [b,H,P,N] they are (0, 1).
    A slice whose reference is all zero contributes its absolute error instead.
    """
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    keep = list(slice_axes)
    red = tuple(i for i in range(got.ndim) if i not in keep)
    err = np.abs(got - ref).max(axis=red) if red else np.abs(got - ref)
    den = np.abs(ref).max(axis=red) if red else np.abs(ref)
    rel = np.where(den > 0, err / np.where(den > 0, den, 1.0), err)
    if np.isnan(got).any():
        return float("inf")
    return float(rel.max())


def rel_y(got, ref):
    return max_rel_err(got, ref, (0, 2))


def rel_h(got, ref):
    return max_rel_err(got, ref, (0, 1))
