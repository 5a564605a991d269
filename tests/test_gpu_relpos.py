"""Bucketed position bias (T5) and relative key/value embeddings (Shaw) on
the GPU, against the f64 oracle, on every path (decode, both prefill
variants, generic)."""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import oracle
import workloads
from gqa_scaled_dot_amd import _lib
from tests.parity import assert_close, dev, torch
from tests.test_oracle_relpos import t5_thresholds

pytestmark = pytest.mark.gpu

PATHS = {"decode": _lib.ATTN_PATH_DECODE, "prefill": _lib.ATTN_PATH_PREFILL,
         "generic": _lib.ATTN_PATH_GENERIC}


def _pb(H, bidirectional=False, nb=32, md=128, seed=11):
    th = t5_thresholds(nb, md, bidirectional)
    rows = len(th) * (2 if bidirectional else 1)
    return th, workloads.normal((rows, H), seed, 3)


def _run(w, q, k, v, bias, params, path=None, variant=0):
    try:
        if path:
            ga.attn_set_option("force_path", PATHS[path])
        ga.attn_set_option("prefill_variant", variant)
        out = ga.attn_forward(dev(q), dev(k), dev(v), dev(bias), **params)
        torch().cuda.synchronize()
        return out.cpu().numpy()
    finally:
        ga.attn_set_option("force_path", 0)
        ga.attn_set_option("prefill_variant", 0)


def _check_pb(w, th, weight, bidirectional, paths, variant=0, rows=None):
    q, k, v, bias = w.tensors()
    wd = dev(weight)
    params = dict(w.params(), position_bias=dict(weight=wd, buckets=th, bidirectional=bidirectional))
    ref = oracle.attention(q, k, v, bias, rows=rows, **w.params(),
                           position_bias=dict(weight=weight, buckets=th, bidirectional=bidirectional))
    for path in paths:
        got = _run(w, q, k, v, bias, params, path, variant)
        sel = got if rows is None else got[np.asarray(rows)]
        assert_close(sel, ref, f"{w.name} {path} v{variant}")


@pytest.mark.parametrize("D, H, G", [(128, 32, 8), (64, 8, 8), (192, 16, 16), (256, 8, 4)])
def test_position_bias_decode(D, H, G):
    w = workloads.Workload("pb decode", T=1, S=3000, heads=H, kvHeads=G, headDim=D,
                           vHeadDim=128 if D == 192 else None, posOffset=2999, seed=D)
    th, weight = _pb(H)
    _check_pb(w, th, weight, False, ("decode", "generic"))


@pytest.mark.parametrize("variant", [32, 16])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("causal, bidirectional", [(True, False), (False, True), (False, False)])
def test_position_bias_prefill(variant, D, causal, bidirectional):
    w = workloads.Workload("pb prefill", T=200, S=260 if causal else 250, heads=8, kvHeads=4, headDim=D,
                           posOffset=60 if causal else 25, causal=causal, seed=D + variant)
    th, weight = _pb(8, bidirectional)
    _check_pb(w, th, weight, bidirectional, ("prefill",), variant)


@pytest.mark.parametrize("features", [dict(softcap=30.0), dict(alibi=True), dict(window=64, sinks=3),
                                      dict(bias="HTS", bias_mask_prob=0.1)])
def test_position_bias_with_other_terms(features):
    w = workloads.Workload("pb mix", T=1, S=700, heads=8, kvHeads=2, headDim=128, posOffset=699, **features)
    th, weight = _pb(8)
    _check_pb(w, th, weight, False, ("decode", "prefill", "generic"))


def test_position_bias_small_tables():
    # One bucket, then thresholds [0, 1, 2, 4, 8, 16] bidirectional on a non-causal decode.
    w = workloads.Workload("pb small", T=2, S=50, heads=4, kvHeads=2, headDim=64, posOffset=20, causal=False)
    _check_pb(w, [0], workloads.normal((1, 4), 2, 3), False, ("decode", "prefill", "generic"))
    _check_pb(w, [0, 1, 2, 4, 8, 16], workloads.normal((12, 4), 3, 3), True, ("decode", "prefill", "generic"))


def test_position_bias_llama_prefill_full_size_sampled():
    w = workloads.LLAMA_PREFILL
    th, weight = _pb(w.heads)
    from tests.parity import sample_rows
    _check_pb(w, th, weight, False, (None,), rows=sample_rows(w.T, seed=3, n_random=8))


def test_position_bias_refusals():
    w = workloads.Workload("pb bad", T=1, S=10, heads=2, headDim=64, posOffset=9)
    q, k, v, _ = w.tensors()
    wt = dev(np.zeros((3, 2), np.float32))
    for buckets, word in (([1, 2, 3], "first threshold"), ([0, 2, 2], "ascend"), ([0, 600, 700], "thresholds past")):
        with pytest.raises(ga.AttnError) as ei:
            ga.attn_forward(dev(q), dev(k), dev(v), **w.params(), position_bias=dict(weight=wt, buckets=buckets))
        assert "position_bias" in ei.value.message and word in ei.value.message


# --------------------------------------------------------------------------
# relative_kv
# --------------------------------------------------------------------------

def _check_rkv(w, m, with_v, paths, seed=21, rows=None):
    q, k, v, bias = w.tensors()
    rk = workloads.normal((2 * m + 1, w.headDim), seed, 1)
    rv = workloads.normal((2 * m + 1, w.Dv), seed, 2) if with_v else None
    params = dict(w.params(), relative_kv=dict(key=dev(rk), value=dev(rv) if with_v else None, max_distance=m))
    ref = oracle.attention(q, k, v, bias, rows=rows, **w.params(),
                           relative_kv=dict(key=rk, value=rv, max_distance=m))
    for path in paths:
        got = _run(w, q, k, v, bias, params, path)
        sel = got if rows is None else got[np.asarray(rows)]
        assert_close(sel, ref, f"{w.name} m={m} {path}")


@pytest.mark.parametrize("D, H, G", [(128, 32, 8), (64, 8, 8), (192, 16, 16), (256, 8, 4)])
@pytest.mark.parametrize("m", [0, 1, 16, 200])
def test_relative_kv_decode(D, H, G, m):
    w = workloads.Workload("rkv decode", T=1, S=3000, heads=H, kvHeads=G, headDim=D,
                           vHeadDim=128 if D == 192 else None, posOffset=2999, seed=D + m)
    _check_rkv(w, m, True, ("decode", "generic"))


@pytest.mark.parametrize("kw", [dict(T=2, heads=8, kvHeads=4), dict(T=1, causal=False, posOffset=900),
                                dict(T=1, softcap=20.0, alibi=True), dict(T=1, window=300, sinks=2),
                                dict(T=4, heads=4, kvHeads=4, posOffset=500)])
def test_relative_kv_decode_features(kw):
    base = dict(T=1, S=1200, heads=8, kvHeads=2, headDim=128, posOffset=1200 - kw.get("T", 1))
    base.update(kw)
    w = workloads.Workload("rkv mix", **base)
    _check_rkv(w, 24, True, ("decode", "generic"))
    _check_rkv(w, 24, False, ("decode",))


def test_relative_kv_forced_splits():
    w = workloads.Workload("rkv splits", T=1, S=5000, heads=8, kvHeads=2, headDim=128, posOffset=4999)
    try:
        for splits in (1, 3, 40):
            ga.attn_set_option("decode_splits", splits)
            _check_rkv(w, 100, True, (None,))
    finally:
        ga.attn_set_option("decode_splits", 0)


def test_relative_kv_prefill_shape_takes_generic():
    w = workloads.Workload("rkv prefill", T=70, S=90, heads=4, kvHeads=2, headDim=64, posOffset=20)
    assert ga.attn_plan(w.T, w.S, **w.params(), relative_kv=dict(key=1, value=None, max_distance=4))["path"] == "generic"
    _check_rkv(w, 4, True, (None,))


def test_relative_kv_refusals():
    w = workloads.Workload("rkv bad", T=1, S=10, heads=2, headDim=64, posOffset=9)
    q, k, v, _ = w.tensors()
    with pytest.raises(ga.AttnError) as ei:
        ga.attn_forward(dev(q), dev(k), dev(v), **w.params(),
                        relative_kv=dict(key=dev(np.zeros((1025 * 2 + 1, 64), np.float32)), max_distance=1025))
    assert "relative_kv" in ei.value.message
