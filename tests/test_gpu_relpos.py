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


@pytest.mark.parametrize("D, H, G", [(128, 32, 8), (128, 64, 8), (64, 8, 8), (192, 16, 16), (256, 8, 4)])
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


@pytest.mark.parametrize("variant", [32, 16])
@pytest.mark.parametrize("S, causal, bidirectional", [(300, True, False), (298, True, False), (260, False, True)])
def test_position_bias_prefill_with_bias_and_alibi(variant, S, causal, bidirectional):
    # The prefill kernels' table lookups beside the bias input's entries,
    # read four per load (S a multiple of 4) or one per load, and ALiBi;
    # 8 heads over 2 KV heads: four heads per workgroup, each its own
    # weights.
    w = workloads.Workload("pb+bias prefill", T=120, S=S, heads=8, kvHeads=2, headDim=128,
                           posOffset=S - 120 if causal else 10, causal=causal, alibi=True, bias="HTS",
                           bias_mask_prob=0.1, seed=S + variant)
    th, weight = _pb(8, bidirectional)
    _check_pb(w, th, weight, bidirectional, ("prefill",), variant)


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


@pytest.mark.parametrize("D, H, G", [(128, 32, 8), (128, 64, 8), (64, 8, 8), (192, 16, 16), (256, 8, 4)])
@pytest.mark.parametrize("m", [0, 1, 16, 200])
def test_relative_kv_decode(D, H, G, m):
    w = workloads.Workload("rkv decode", T=1, S=3000, heads=H, kvHeads=G, headDim=D,
                           vHeadDim=128 if D == 192 else None, posOffset=2999, seed=D + m)
    _check_rkv(w, m, True, ("decode", "generic"))


@pytest.mark.parametrize("kw", [dict(T=2, heads=8, kvHeads=4), dict(T=2, heads=16, kvHeads=4),
                                dict(T=1, causal=False, posOffset=900),
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


def _rkv_plan(w, m):
    return ga.attn_plan(w.T, w.S, bias_kind={None: 0, "TS": 1, "HTS": 2}[w.bias], **w.params(),
                        relative_kv=dict(key=1, value=None, max_distance=m))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("m", [0, 1, 16, 40, 200])
def test_relative_kv_prefill(D, causal, m):
    # The 32x32x2 prefill kernel with relative embeddings: keys far on either
    # side of each query (one embedding row each) and the band within m of it
    # (per-key rows), on ragged tiles; also without value embeddings; and the
    # generic kernel on the same call.
    w = workloads.Workload("rkv prefill", T=150, S=230 if causal else 200, heads=8, kvHeads=2, headDim=D,
                           posOffset=80 if causal else 30, causal=causal, seed=D + m)
    assert _rkv_plan(w, m)["path"] == "prefill"
    _check_rkv(w, m, True, (None, "generic"), seed=m)
    _check_rkv(w, m, False, (None,), seed=m + 1)


@pytest.mark.parametrize("kw", [dict(window=50, sinks=3), dict(causal=False, window=40, posOffset=60),
                                dict(softcap=20.0, alibi=True, bias="HTS", bias_mask_prob=0.1, std=2.0),
                                dict(T=300, S=300, posOffset=0, heads=4, kvHeads=4),
                                dict(T=70, S=900, posOffset=830)])
def test_relative_kv_prefill_features(kw):
    base = dict(T=160, S=400, heads=8, kvHeads=2, headDim=128, posOffset=240)
    base.update(kw)
    w = workloads.Workload("rkv prefill mix", **base)
    q, k, v, bias = w.tensors()
    assert _rkv_plan(w, 32)["path"] == "prefill"
    _check_rkv(w, 32, True, (None,), seed=5)


@pytest.mark.parametrize("splits", [2, 5])
def test_relative_kv_prefill_key_splits(splits):
    # Key-range parts merged by the combine kernel: the embedding terms and
    # the far-key weight sums travel in the partial states.
    w = workloads.Workload("rkv prefill splits", T=100, S=2000, heads=8, kvHeads=2, headDim=128, posOffset=1900)
    try:
        ga.attn_set_option("prefill_splits", splits)
        # At 128-wide heads the band tiles take a launch (and a partial) of their own.
        assert _rkv_plan(w, 64)["splits"] == splits + 1
        _check_rkv(w, 64, True, (None,), seed=splits)
    finally:
        ga.attn_set_option("prefill_splits", 0)


def test_relative_kv_wide_heads_take_generic():
    # 192/128 and 256 widths have no prefill instance with the embeddings.
    for D, Dv in ((192, 128), (256, 256)):
        w = workloads.Workload("rkv wide", T=70, S=90, heads=4, kvHeads=2, headDim=D, vHeadDim=Dv, posOffset=20)
        assert _rkv_plan(w, 4)["path"] == "generic"
    _check_rkv(w, 4, True, (None,))


def test_relative_kv_chunked_prefill_full_size_sampled():
    # The Llama-shaped chunked prefill (T=512 at 3584 over 4096 keys) with
    # relative embeddings of max distance 128, sampled rows.
    from tests.parity import sample_rows
    w = workloads.LLAMA_CHUNKED
    assert _rkv_plan(w, 128)["path"] == "prefill"
    _check_rkv(w, 128, True, (None,), rows=sample_rows(w.T, seed=4, n_random=24, edges=(128, 256)))


def test_relative_kv_refusals():
    w = workloads.Workload("rkv bad", T=1, S=10, heads=2, headDim=64, posOffset=9)
    q, k, v, _ = w.tensors()
    with pytest.raises(ga.AttnError) as ei:
        ga.attn_forward(dev(q), dev(k), dev(v), **w.params(),
                        relative_kv=dict(key=dev(np.zeros((1025 * 2 + 1, 64), np.float32)), max_distance=1025))
    assert "relative_kv" in ei.value.message
