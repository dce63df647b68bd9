"""Comparison of fp16 GPU outputs with the fp64 oracle.

The bar (both must hold): max |gpu - oracle| <= 2e-3 and
||gpu - oracle||_2 / ||oracle||_2 <= 1e-3.  Cosine similarity, mean absolute
error and the fraction of elements within one fp16 ULP of the oracle are
reported beside them, in the styles the pages use for their operator checks.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = 2e-3
REL_L2 = 1e-3


def metrics(got: np.ndarray, ref: np.ndarray) -> dict:
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    d = g - r
    nr = np.linalg.norm(r)
    ulp = np.spacing(np.abs(r).astype(np.float16)).astype(np.float64)
    return dict(
        max_abs=float(np.abs(d).max()) if d.size else 0.0,
        rel_l2=float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d)),
        cosine=float(np.dot(g.ravel(), r.ravel()) / (np.linalg.norm(g) * nr)) if nr > 0 else 1.0,
        mae=float(np.abs(d).mean()) if d.size else 0.0,
        within_1ulp=float(np.mean(np.abs(d) <= ulp)) if d.size else 1.0,
        finite=bool(np.isfinite(g).all()),
    )


def assert_parity(got, ref, what: str = "", max_abs: float = MAX_ABS, rel_l2: float = REL_L2) -> dict:
    m = metrics(got, ref)
    print(f"[parity] {what}: " + " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                         for k, v in m.items()), flush=True)
    assert m["finite"], f"{what}: non-finite output"
    assert m["max_abs"] <= max_abs, f"{what}: max abs {m['max_abs']:.3e} > {max_abs}"
    assert m["rel_l2"] <= rel_l2, f"{what}: rel L2 {m['rel_l2']:.3e} > {rel_l2}"
    return m
