"""Seeded random combinations of the op's features on every path, against the oracle.

Each case draws a shape (head widths with and without matrix-core
instances, grouped-query ratios of 1 to 8 query heads per KV head, one to a
few dozen query rows) and a mix of
the op's parameters (causal or not, posOffset, window with or without sinks,
softcap, the three ALiBi forms, either bias layout, a scale override), then
runs it on the path the library picks and again on every other path the
`force_path` option can force for that call. Sizes stay small so
the oracle computes every row. Same bar as everywhere: |gpu - ref| <= 1e-4 +
1e-4 |ref|.
"""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import workloads
from gqa_scaled_dot_amd import _lib
from tests.parity import compare

pytestmark = pytest.mark.gpu

N_CASES = 150
N_WIDE_CASES = 50  # further cases with 5 to 8 query heads per KV head
PATHS = {"generic": _lib.ATTN_PATH_GENERIC, "decode": _lib.ATTN_PATH_DECODE, "prefill": _lib.ATTN_PATH_PREFILL}
WIDTHS = [(64, 64), (128, 128), (192, 128), (256, 256), (32, 32), (80, 48)]


def _draw(i: int) -> workloads.Workload:
    r = np.random.default_rng(np.random.SeedSequence([2024, i]))
    D, Dv = WIDTHS[r.integers(len(WIDTHS))]
    G = int(r.choice([1, 2, 4, 8]))
    wide = N_CASES <= i < N_CASES + N_WIDE_CASES
    hpg = int(r.choice([5, 6, 7, 8])) if wide else int(r.choice([1, 2, 4]))
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


@pytest.mark.parametrize("i", range(N_CASES + N_WIDE_CASES))
def test_random_combination(i):
    w = _draw(i)
    q, k, v, bias = w.tensors()
    params = w.params()
    kind = {None: 0, "TS": 1, "HTS": 2}[w.bias]
    auto = ga.attn_plan(w.T, w.S, bias_kind=kind, **params)["path"]
    compare(q, k, v, bias, params, what=f"{w} (auto: {auto})")
    # Every other path that can take the call.
    others = [p for p in ("decode", "prefill", "generic") if p != auto]
    for other in others:
        try:
            ga.attn_set_option("force_path", PATHS[other])
            try:
                planned = ga.attn_plan(w.T, w.S, bias_kind=kind, **params)["path"]
            except ga.AttnError:
                continue  # that path has no kernel for this shape
            assert planned in (other, "zero"), (other, planned)
            compare(q, k, v, bias, params, what=f"{w} (forced {other})")
        finally:
            ga.attn_set_option("force_path", 0)


N_TERM_CASES = 60


def _terms(i: int, w: workloads.Workload):
    """A bucketed position bias or relative key/value embeddings for w (host arrays)."""
    r = np.random.default_rng(np.random.SeedSequence([2025, i]))
    if r.random() < 0.5:
        n = int(r.integers(2, 40))
        th = [0] + sorted(int(x) for x in r.choice(np.arange(1, 513), n - 1, replace=False))
        bidir = bool(r.random() < 0.5)
        weight = workloads.normal((n * (2 if bidir else 1), w.heads), 300 + i, 3)
        return "position_bias", dict(weight=weight, buckets=th, bidirectional=bidir)
    m = int(r.integers(1, 200))
    rk = workloads.normal((2 * m + 1, w.headDim), 300 + i, 5)
    rv = workloads.normal((2 * m + 1, w.Dv), 300 + i, 6) if r.random() < 0.7 else None
    return "relative_kv", dict(key=rk, value=rv, max_distance=m)


@pytest.mark.parametrize("i", range(N_TERM_CASES))
def test_random_combination_with_relative_terms(i):
    from tests.parity import assert_close, dev, torch
    import oracle
    w = _draw(1000 + i)
    name, term = _terms(i, w)
    q, k, v, bias = w.tensors()
    dterm = {kk: (dev(vv) if isinstance(vv, np.ndarray) else vv) for kk, vv in term.items()}
    ref = oracle.attention(q, k, v, bias, **w.params(), **{name: term})
    kind = {None: 0, "TS": 1, "HTS": 2}[w.bias]
    params = dict(w.params(), **{name: dterm})
    auto = ga.attn_plan(w.T, w.S, bias_kind=kind, **params)["path"]
    for path in [None] + [p for p in ("decode", "prefill", "generic") if p != auto]:
        try:
            if path:
                ga.attn_set_option("force_path", PATHS[path])
                try:
                    planned = ga.attn_plan(w.T, w.S, bias_kind=kind, **params)["path"]
                except ga.AttnError:
                    continue
                assert planned in (path, "zero"), (path, planned)
            got = ga.attn_forward(dev(q), dev(k), dev(v), dev(bias), **params)
            torch().cuda.synchronize()
            assert_close(got.cpu().numpy(), ref, f"{w} {name} ({path or 'auto: ' + auto})")
        finally:
            ga.attn_set_option("force_path", 0)


MLA_SHAPES = [(512, 64, 128, 128), (256, 64, 128, 128), (512, 64, 64, 96), (48, 16, 24, 20), (96, 0, 32, 16)]


@pytest.mark.parametrize("i", range(40))
def test_random_mla_combination(i):
    from tests.parity import assert_close, dev, torch
    from oracle import mla
    r = np.random.default_rng(np.random.SeedSequence([2026, i]))
    R, P, N, Dv = MLA_SHAPES[r.integers(len(MLA_SHAPES))]
    H = int(r.choice([1, 3, 16, 20, 40]))
    T = int(r.choice([1, 1, 2, 5, 17]))
    S = int(r.integers(max(T, 1), 900))
    causal = bool(r.random() < 0.7)
    pos = (S - T if r.random() < 0.6 else int(r.integers(0, S - T + 1))) if causal else int(r.integers(0, S + 1))
    kw = dict(name=f"mla combination {i}", T=T, S=S, heads=H, kv_rank=R, qk_nope=N, qk_rope=P, v_head_dim=Dv,
              causal=causal, posOffset=pos, seed=500 + i)
    if r.random() < 0.5:
        kw["window"] = int(r.integers(1, S + 1))
        if r.random() < 0.5:
            kw["sinks"] = int(r.integers(1, 9))
    if r.random() < 0.3:
        kw["scale"] = float(np.float32(r.uniform(0.02, 0.2)))
    w = workloads.MlaWorkload(**kw)
    q, state, k_b, v_b = w.tensors()
    ref = mla.mla_attention(q, state, k_b, v_b, **w.params())
    for generic in (0, 1):
        try:
            ga.attn_set_option("mla_generic", generic)
            got = ga.attn_mla_forward(dev(q), dev(state), dev(k_b), dev(v_b), **w.params())
            torch().cuda.synchronize()
        finally:
            ga.attn_set_option("mla_generic", 0)
        assert_close(got.cpu().numpy(), ref, f"{w} generic={generic}")
