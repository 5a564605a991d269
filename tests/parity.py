"""Helpers for the GPU parity tests: run the HIP library and the oracle on
the same seeded inputs and compare element by element.

Bar (f32 result against the f64 oracle): |gpu - ref| <= 1e-4 + 1e-4 * |ref|
for every element; cache_write must match bit for bit.
"""

from __future__ import annotations

import numpy as np

import oracle

ATOL = 1e-4
RTOL = 1e-4


def torch():
    import torch as _t
    return _t


def dev(x):
    if x is None:
        return None
    return torch().from_numpy(np.ascontiguousarray(x)).to("cuda")


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    """Check the bar; return the largest |err| / (ATOL + RTOL |ref|)."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    ratio = err / bound
    worst = np.unravel_index(np.argmax(ratio), ratio.shape) if ratio.size else ()
    if ratio.size and ratio[worst] > 1.0:
        raise AssertionError(
            f"{what}: |err| {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst} "
            f"(got {got[worst]!r}, ref {ref[worst]!r}); {int((ratio > 1).sum())} elements out")
    return float(ratio.max()) if ratio.size else 0.0


def run_library(q, k, v, bias, params, *, out=None):
    import gqa_scaled_dot_amd as ga
    t = torch()
    res = ga.attn_forward(dev(q) if isinstance(q, np.ndarray) else q,
                          dev(k) if isinstance(k, np.ndarray) else k,
                          dev(v) if isinstance(v, np.ndarray) else v,
                          dev(bias) if isinstance(bias, np.ndarray) else bias,
                          out=out, **params)
    t.cuda.synchronize()
    return res


def compare(q, k, v, bias, params, *, rows=None, what="", out=None):
    """Run both sides; compare all rows or the listed ones. Returns the GPU output (numpy)."""
    got = run_library(q, k, v, bias, params, out=out).cpu().numpy()
    ref = oracle.attention(q, k, v, bias, rows=rows, **params)
    sel = got if rows is None else got[np.asarray(rows)]
    assert_close(sel, ref, what)
    return got


def sample_rows(T: int, seed: int = 0, n_random: int = 48, edges=()):
    """First and last 16 rows, rows around the given edge positions, and seeded random rows."""
    rows = set(range(min(16, T))) | set(range(max(0, T - 16), T))
    for e in edges:
        for r in range(e - 3, e + 4):
            if 0 <= r < T:
                rows.add(r)
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.integers(0, T, size=min(n_random, T)))
    return sorted(rows)
