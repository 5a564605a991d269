"""Prefill path (fp32 MFMA flash kernel) against the oracle, on the GPU."""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
from gqa_scaled_dot_amd import _lib
import oracle
import workloads
from tests.parity import assert_close, compare, dev, run_library, sample_rows, torch

pytestmark = pytest.mark.gpu

BIAS_KIND = {None: 0, "TS": 1, "HTS": 2}


@pytest.fixture(params=[32, 16], ids=["mfma32", "mfma16"])
def variant(request):
    """Run a test on both prefill kernels (32x32x2 and 16x16x4 MFMA)."""
    ga.attn_set_option("prefill_variant", request.param)
    yield request.param
    ga.attn_set_option("prefill_variant", 0)


def _check(w, rows=None, what=None, path="prefill"):
    q, k, v, bias = w.tensors()
    params = w.params()
    plan = ga.attn_plan(w.T, w.S, bias_kind=BIAS_KIND[w.bias], **params)
    assert plan["path"] == path, plan
    return compare(q, k, v, bias, params, rows=rows, what=what or w.name)


# Head layouts: heads per KV group 4 (4 heads side by side), 8 (two head
# groups), 2 (2 heads x 2 query blocks), 1 (4 query blocks), 3 (1 head x 4).
@pytest.mark.parametrize("D, Dv", [(64, 64), (128, 128), (192, 128), (256, 256)])
@pytest.mark.parametrize("H, G", [(8, 2), (8, 1), (4, 2), (4, 4), (6, 2)])
def test_prefill_shapes_ragged(D, Dv, H, G, variant):
    w = workloads.Workload("prefill shape", T=100, S=100, heads=H, kvHeads=G, headDim=D, vHeadDim=Dv,
                           seed=D + 7 * H + G)
    _check(w)


@pytest.mark.parametrize("feature", [
    dict(), dict(causal=False), dict(window=37), dict(window=1), dict(causal=False, window=20),
    dict(softcap=5.0, std=3.0), dict(alibi=True), dict(alibiMax=4.0),
    dict(alibiSlopes=tuple(0.02 * (h + 1) for h in range(8))), dict(scale=0.05),
    dict(bias="TS", bias_mask_prob=0.1), dict(bias="HTS", bias_mask_prob=0.3),
    dict(causal=False, bias="HTS", bias_mask_prob=0.1, alibi=True),
    dict(softcap=10.0, window=50, alibi=True, bias="HTS", bias_mask_prob=0.1, std=2.0),
])
@pytest.mark.parametrize("D, Dv", [(128, 128), (256, 256), (192, 128)])
def test_prefill_features(feature, D, Dv, variant):
    w = workloads.Workload("prefill features", T=150, S=150, heads=8, kvHeads=2, headDim=D, vHeadDim=Dv,
                           **feature)
    q, k, v, bias = w.tensors()
    if bias is not None:
        bias[..., 0] = 0.0  # key 0 stays unmasked (causal rows always see it)
    compare(q, k, v, bias, w.params(), what=f"{feature} D={D}")


@pytest.mark.parametrize("T, S, P0", [(64, 200, 136), (33, 90, 57), (1, 300, 299), (200, 64, 0),
                                      (70, 400, 100)])
def test_prefill_pos_offset_and_rectangles(T, S, P0, variant):
    # Chunked prefill against a longer cache (rows past P0+T-1 may hold anything).
    w = workloads.Workload("chunked", T=T, S=S, heads=8, kvHeads=2, headDim=128, posOffset=P0)
    q, k, v, _ = w.tensors()
    if P0 + T < S:
        k[P0 + T:] = np.nan
        v[P0 + T:] = np.nan
    try:
        ga.attn_set_option("force_path", _lib.ATTN_PATH_PREFILL)
        got = compare(q, k, v, None, w.params(), what=f"T={T} S={S} P0={P0}")
    finally:
        ga.attn_set_option("force_path", 0)
    assert np.isfinite(got).all()


def test_prefill_window_never_reads_outside(variant):
    # Keys before every row's window are NaN: they must not be read.
    w = workloads.Workload("window", T=64, S=300, heads=8, kvHeads=2, headDim=128, posOffset=236,
                           window=40)
    q, k, v, _ = w.tensors()
    k[:236 - 40] = np.nan
    v[:236 - 40] = np.nan
    compare(q, k, v, None, w.params(), what="window with NaN before it")


def test_prefill_empty_rows_are_zero(variant):
    # Non-causal window where the last rows see nothing (keys end at 10).
    w = workloads.Workload("empty rows", T=40, S=10, heads=4, kvHeads=4, headDim=128, causal=False,
                           window=3)
    q, k, v, _ = w.tensors()
    got = compare(q, k, v, None, w.params(), what="empty rows")
    assert np.all(got[14:] == 0.0)


def test_prefill_matches_decode_and_generic():
    w = workloads.Workload("three paths", T=1, S=2000, heads=8, kvHeads=2, headDim=128, posOffset=1999,
                           alibi=True, softcap=20.0)
    q, k, v, _ = w.tensors()
    outs = {}
    try:
        for name, path in (("decode", _lib.ATTN_PATH_DECODE), ("prefill", _lib.ATTN_PATH_PREFILL),
                           ("generic", _lib.ATTN_PATH_GENERIC)):
            ga.attn_set_option("force_path", path)
            outs[name] = compare(q, k, v, None, w.params(), what=name)
    finally:
        ga.attn_set_option("force_path", 0)
    np.testing.assert_allclose(outs["prefill"], outs["decode"], rtol=2e-4, atol=2e-4)


def test_prefill_is_deterministic():
    w = workloads.Workload("determinism", T=300, S=300, heads=8, kvHeads=2, headDim=128, alibi=True)
    q, k, v, _ = w.tensors()
    a = run_library(q, k, v, None, w.params()).cpu().numpy()
    b = run_library(q, k, v, None, w.params()).cpu().numpy()
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


# ---- full-size workloads, sampled rows --------------------------------------

def test_llama_prefill_full_size_sampled(variant):
    w = workloads.LLAMA_PREFILL
    _check(w, rows=sample_rows(w.T, seed=1, n_random=40, edges=(2048,)))


def test_llama_chunked_prefill_full_size():
    w = workloads.LLAMA_CHUNKED
    _check(w, rows=sample_rows(w.T, seed=2, n_random=64))


def test_gemma2_swa_full_size_sampled(variant):
    w = workloads.GEMMA2_SWA
    _check(w, rows=sample_rows(w.T, seed=3, n_random=24, edges=(4095, 4096, 4097, 6000)))


def test_latent_noncausal_full_size(variant):
    w = workloads.LATENT_NONCAUSAL
    _check(w, rows=sample_rows(w.T, seed=4, n_random=64))


@pytest.mark.parametrize("splits", [2, 3, 7])
def test_prefill_key_splits_match(splits, variant):
    # Forced key-range splits (merged by the combine kernel) give the same result.
    w = workloads.Workload("split prefill", T=70, S=500, heads=8, kvHeads=2, headDim=128, posOffset=430,
                           alibi=True)
    q, k, v, _ = w.tensors()
    try:
        ga.attn_set_option("prefill_splits", splits)
        assert ga.attn_plan(w.T, w.S, **w.params())["splits"] == splits
        compare(q, k, v, None, w.params(), what=f"prefill splits={splits}")
    finally:
        ga.attn_set_option("prefill_splits", 0)


@pytest.mark.parametrize("window", [1000, 2 ** 31 - 1, 2 ** 40])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_windows_wider_than_any_distance(window, causal, variant):
    # Windows at and past 2^31 - 1: a window that cannot hide a key must give
    # the result without one (no position + window sum may wrap), and one that
    # still hides keys (1000 of 1023 distances) must keep hiding them.
    w = workloads.Workload("wide window", T=1024, S=1024, heads=8, kvHeads=2, headDim=128,
                           causal=causal, window=window, seed=window % 997)
    _check(w, rows=sample_rows(w.T, seed=3, edges=(1000, 23)), what=f"window={window} causal={causal}")


@pytest.mark.parametrize("S", [260, 258], ids=["rows16B", "ragged"])
@pytest.mark.parametrize("kind, causal", [("TS", True), ("HTS", False)])
@pytest.mark.parametrize("D, Dv", [(128, 128), (192, 128)])
def test_prefill_bias_entries_four_at_a_time(S, kind, causal, D, Dv, variant):
    # Bias rows of a multiple of 4 entries are read four entries per load;
    # ragged rows (S not a multiple of 4) one entry per load. Both against the
    # oracle, with ALiBi beside the bias and a last key tile past S.
    w = workloads.Workload("bias four at a time", T=96, S=S, heads=8, kvHeads=2, headDim=D, vHeadDim=Dv,
                           causal=causal, posOffset=S - 96 if causal else 0, alibi=True, bias=kind,
                           bias_mask_prob=0.1, seed=S + D)
    q, k, v, bias = w.tensors()
    compare(q, k, v, bias, w.params(), what=f"{kind} S={S} D={D}")


@pytest.mark.parametrize("T, H, G", [(2048, 32, 32), (1024, 28, 4), (4096, 40, 8)])
def test_causal_prefill_split_plans_sampled(T, H, G):
    # Causal MHA and 7- or 5-heads-per-KV-head shapes (one head per
    # workgroup) take key-split plans of 2-4 parts: sampled rows, the
    # diagonal's included, against the oracle.
    w = workloads.Workload("causal split plan", T=T, S=T, heads=H, kvHeads=G, headDim=128, seed=T + H)
    plan = ga.attn_plan(w.T, w.S, **w.params())
    assert plan["path"] == "prefill" and plan["splits"] > 1, plan
    _check(w, rows=sample_rows(w.T, seed=H, n_random=24, edges=(w.T // 2, 127, 128)))
