"""Seeded random combinations of the op's features on every path, against the oracle.

Each case draws a shape (head widths with and without matrix-core
instances, grouped-query ratios, one to a few dozen query rows) and a mix of
the op's parameters (causal or not, posOffset, window with or without sinks,
softcap, the three ALiBi forms, either bias layout, a scale override), then
runs it on the path the library picks and again on a path forced by the
`force_path` option where that path can serve the call. Sizes stay small so
the oracle computes every row. Same bar as everywhere: |gpu - ref| <= 1e-4 +
1e-4 |ref|.
"""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import workloads
from tests.parity import compare

pytestmark = pytest.mark.gpu

N_CASES = 150
PATHS = {"generic": 1, "decode": 2, "prefill": 3}  # ATTN_PATH_GENERIC / _DECODE / _PREFILL
WIDTHS = [(64, 64), (128, 128), (192, 128), (256, 256), (32, 32), (80, 48)]


def _draw(i: int) -> workloads.Workload:
    r = np.random.default_rng(np.random.SeedSequence([2024, i]))
    D, Dv = WIDTHS[r.integers(len(WIDTHS))]
    G = int(r.choice([1, 2, 4, 8]))
    hpg = int(r.choice([1, 2, 4]))
    H = G * hpg
    T = int(r.choice([1, 1, 2, 3, int(r.integers(5, 70))]))
    S = int(r.integers(max(T, 1), 700))
    causal = bool(r.random() < 0.7)
    if causal:
        # Rows at the cache's end, or earlier with unwritten rows past them.
        pos = S - T if r.random() < 0.6 else int(r.integers(0, S - T + 1))
    else:
        pos = int(r.integers(0, S + 1))
    kw = dict(name=f"combination {i}", T=T, S=S, heads=H, kvHeads=G, headDim=D, vHeadDim=Dv,
              causal=causal, posOffset=pos, seed=100 + i)
    if r.random() < 0.5:
        kw["window"] = int(r.integers(1, S + 1))
        if r.random() < 0.5:
            kw["sinks"] = int(r.integers(1, 9))
    if r.random() < 0.35:
        kw["softcap"] = float(np.float32(r.uniform(5.0, 50.0)))
        kw["std"] = 2.0
    alibi = r.integers(4)
    if alibi == 1:
        kw["alibi"] = True
    elif alibi == 2:
        kw["alibiMax"] = 8.0
    elif alibi == 3:
        kw["alibiSlopes"] = tuple(float(np.float32(x)) for x in r.uniform(0.001, 0.3, H))
    b = r.integers(3)
    if b:
        kw["bias"] = "TS" if b == 1 else "HTS"
        kw["bias_mask_prob"] = float(r.choice([0.0, 0.1, 0.5]))
    if r.random() < 0.3:
        kw["scale"] = float(np.float32(r.uniform(0.02, 0.3)))
    return workloads.Workload(**kw)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_combination(i):
    w = _draw(i)
    q, k, v, bias = w.tensors()
    params = w.params()
    kind = {None: 0, "TS": 1, "HTS": 2}[w.bias]
    auto = ga.attn_plan(w.T, w.S, bias_kind=kind, **params)["path"]
    compare(q, k, v, bias, params, what=f"{w} (auto: {auto})")
    # One other path that can take the call.
    others = [p for p in ("decode", "prefill", "generic") if p != auto]
    for other in others:
        try:
            ga.attn_set_option("force_path", PATHS[other])
            try:
                ga.attn_plan(w.T, w.S, bias_kind=kind, **params)
            except ga.AttnError:
                continue  # that path has no kernel for this shape
            compare(q, k, v, bias, params, what=f"{w} (forced {other})")
            break
        finally:
            ga.attn_set_option("force_path", 0)
