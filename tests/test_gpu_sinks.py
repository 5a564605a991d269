"""Attention sinks beside a sliding window, on the GPU, against the oracle.

With a window on, keys s < sinks stay visible (causal rows: at or before
their position). The keys between the sinks and a row's window are never
read: the tests fill them with NaN, so any read would show in the output.
"""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import oracle
import workloads
from gqa_scaled_dot_amd import _lib
from tests.parity import compare, dev, sample_rows, torch

pytestmark = pytest.mark.gpu

PATHS = {"decode": _lib.ATTN_PATH_DECODE, "prefill": _lib.ATTN_PATH_PREFILL,
         "generic": _lib.ATTN_PATH_GENERIC}


def _poison_gap(k, v, sinks, first_seen):
    """NaN in key rows [sinks, first_seen): no row may read them."""
    if first_seen > sinks:
        k[sinks:first_seen] = np.nan
        v[sinks:first_seen] = np.nan


def _run_paths(w, paths, k=None, v=None, what=""):
    q, k0, v0, bias = w.tensors()
    k = k0 if k is None else k
    v = v0 if v is None else v
    outs = {}
    try:
        for path in paths:
            ga.attn_set_option("force_path", PATHS[path])
            outs[path] = compare(q, k, v, bias, w.params(), what=f"{what} {path}")
    finally:
        ga.attn_set_option("force_path", 0)
    return outs


@pytest.mark.parametrize("D, H, G", [(128, 32, 8), (64, 8, 2), (192, 16, 16), (256, 8, 4)])
@pytest.mark.parametrize("window, sinks", [(512, 4), (64, 1), (300, 100)])
def test_decode_with_sinks_never_reads_the_gap(D, H, G, window, sinks):
    S = 3000
    w = workloads.Workload("decode sinks", T=1, S=S, heads=H, kvHeads=G, headDim=D,
                           vHeadDim=128 if D == 192 else None, posOffset=S - 1, window=window,
                           sinks=sinks, seed=D + window)
    q, k, v, _ = w.tensors()
    _poison_gap(k, v, sinks, S - window)
    plan = ga.attn_plan(w.T, w.S, **w.params())
    assert plan["path"] == "decode"
    _run_paths(w, ("decode", "prefill", "generic") if D != 192 else ("decode", "generic"), k, v,
               what=f"D={D} window={window} sinks={sinks}")


def test_decode_sink_split_and_forced_split_counts():
    w = workloads.Workload("split counts", T=1, S=5000, heads=8, kvHeads=2, headDim=128, posOffset=4999,
                           window=1000, sinks=16, alibi=True, softcap=30.0)
    q, k, v, _ = w.tensors()
    _poison_gap(k, v, 16, 4000)
    try:
        for splits in (1, 2, 7, 16):
            ga.attn_set_option("decode_splits", splits)
            # The window's 1000 keys keep the forced count (chunks of whole
            # 64-key steps, finer where those would drop a split), plus the
            # sink split.
            assert ga.attn_plan(w.T, w.S, **w.params())["splits"] == splits + 1
            compare(q, k, v, None, w.params(), what=f"window splits {splits}")
    finally:
        ga.attn_set_option("decode_splits", 0)


def test_sinks_only_when_the_window_is_past_the_keys():
    # Non-causal rows beyond the cache: the window holds no key, the sinks do.
    w = workloads.Workload("sinks only", T=2, S=40, heads=4, kvHeads=2, headDim=64, posOffset=100,
                           causal=False, window=3, sinks=5)
    outs = _run_paths(w, ("decode", "prefill", "generic"), what="sinks only")
    assert np.isfinite(outs["decode"]).all()


@pytest.mark.parametrize("variant", [32, 16])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("window, sinks, causal", [(50, 4, True), (50, 40, True), (7, 3, True),
                                                   (20, 6, False), (1, 1, True)])
def test_prefill_with_sinks(variant, D, window, sinks, causal):
    T, P0 = 96, 1000
    S = P0 + T if causal else P0 + T + 10
    w = workloads.Workload("prefill sinks", T=T, S=S, heads=8, kvHeads=2, headDim=D, posOffset=P0,
                           window=window, sinks=sinks, causal=causal, seed=window + sinks)
    q, k, v, _ = w.tensors()
    _poison_gap(k, v, sinks, P0 - window)
    try:
        ga.attn_set_option("prefill_variant", variant)
        ga.attn_set_option("force_path", _lib.ATTN_PATH_PREFILL)
        compare(q, k, v, None, w.params(), what=f"v{variant} D={D} w={window} sinks={sinks}")
    finally:
        ga.attn_set_option("prefill_variant", 0)
        ga.attn_set_option("force_path", 0)


@pytest.mark.parametrize("splits", [2, 5])
def test_prefill_key_splits_with_sinks(splits):
    w = workloads.Workload("split prefill sinks", T=70, S=800, heads=8, kvHeads=2, headDim=128,
                           posOffset=730, window=64, sinks=8, alibi=True)
    q, k, v, _ = w.tensors()
    _poison_gap(k, v, 8, 730 - 64)
    try:
        ga.attn_set_option("prefill_splits", splits)
        compare(q, k, v, None, w.params(), what=f"prefill splits {splits}")
    finally:
        ga.attn_set_option("prefill_splits", 0)


def test_prefill_from_position_zero_with_sinks():
    # Early rows have the sinks inside their window; later rows see both.
    w = workloads.Workload("prefill from 0", T=300, S=300, heads=8, kvHeads=4, headDim=128,
                           window=37, sinks=5, softcap=20.0)
    _run_paths(w, ("prefill", "generic"), what="from 0")


def test_gemma2_swa_with_sinks_full_size_sampled():
    w = workloads.GEMMA2_SWA.replace(sinks=4)
    q, k, v, _ = w.tensors()
    rows = sample_rows(w.T, seed=9, n_random=16, edges=(4095, 4096, 4100, 8191))
    compare(q, k, v, None, w.params(), rows=rows, what="gemma2 + sinks")


def test_streaming_decode_full_size():
    w = workloads.LLAMA_STREAMING
    q, k, v, _ = w.tensors()
    _poison_gap(k, v, w.sinks, w.S - w.window)
    got = compare(q, k, v, None, w.params(), what=w.name)
    assert np.isfinite(got).all()
