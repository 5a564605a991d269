"""The any-width correctness path, and the degenerate calls, on the GPU."""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
from gqa_scaled_dot_amd import _lib
import workloads
from tests.parity import compare, dev, run_library, sample_rows, torch

pytestmark = pytest.mark.gpu


def test_tiny_causal_prefill():
    w = workloads.TINY
    q, k, v, _ = w.tensors()
    assert ga.attn_plan(w.T, w.S, **w.params())["path"] == "generic"
    compare(q, k, v, None, w.params(), what=w.name)


@pytest.mark.parametrize("feature", [
    dict(), dict(window=3), dict(causal=False), dict(causal=False, window=2, posOffset=4),
    dict(softcap=2.0, std=3.0), dict(alibi=True), dict(alibiMax=4.0), dict(scale=0.7),
    dict(bias="TS", bias_mask_prob=0.2), dict(bias="HTS", bias_mask_prob=0.2),
    dict(posOffset=5, S=20, window=4, softcap=3.0, alibi=True, bias="HTS", bias_mask_prob=0.1),
])
def test_odd_widths_all_features(feature):
    base = dict(name="odd widths", T=9, S=13, heads=6, kvHeads=3, headDim=3, vHeadDim=5)
    base.update(feature)
    w = workloads.Workload(**base)
    q, k, v, bias = w.tensors()
    if bias is not None:
        bias[..., 0] = 0.0
    compare(q, k, v, bias, w.params(), what=str(feature))


def test_generic_prefill_shape_with_ragged_tail():
    w = workloads.Workload("generic prefill", T=300, S=300, heads=8, kvHeads=2, headDim=128)
    q, k, v, _ = w.tensors()
    compare(q, k, v, None, w.params(), rows=sample_rows(300), what=w.name)


def test_forced_generic_matches_decode():
    w = workloads.Workload("decode shape", T=1, S=3000, heads=32, kvHeads=8, headDim=128,
                           posOffset=2999, alibi=True)
    q, k, v, _ = w.tensors()
    dec = run_library(q, k, v, None, w.params()).cpu().numpy()
    try:
        ga.attn_set_option("force_path", _lib.ATTN_PATH_GENERIC)
        gen = compare(q, k, v, None, w.params(), what="forced generic")
    finally:
        ga.attn_set_option("force_path", 0)
    np.testing.assert_allclose(gen, dec, rtol=2e-4, atol=2e-4)


def test_zero_query_rows_is_a_noop():
    t = torch()
    q = t.zeros((0, 64), dtype=t.float32, device="cuda")
    k = t.zeros((5, 64), dtype=t.float32, device="cuda")
    out = ga.attn_forward(q, k, k, heads=1, headDim=64)
    t.cuda.synchronize()
    assert tuple(out.shape) == (0, 64)


def test_zero_keys_gives_zeros():
    t = torch()
    q = dev(workloads.normal((3, 128), 0, 0))
    k = t.zeros((0, 128), dtype=t.float32, device="cuda")
    out = t.full((3, 128), float("nan"), dtype=t.float32, device="cuda")
    ga.attn_forward(q, k, k, out=out, heads=1, headDim=128)
    t.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0.0)


def test_no_visible_key_anywhere_gives_zeros():
    t = torch()
    q = dev(workloads.normal((2, 128), 0, 0))
    k = dev(workloads.normal((4, 128), 0, 1))
    out = t.full((2, 128), float("nan"), dtype=t.float32, device="cuda")
    ga.attn_forward(q, k, k, out=out, heads=1, headDim=128, posOffset=10, window=2)
    t.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0.0)


def test_invalid_call_writes_nothing():
    t = torch()
    q = dev(workloads.normal((2, 128), 0, 0))
    out = t.full((2, 128), 7.0, dtype=t.float32, device="cuda")
    with pytest.raises(ga.AttnError):
        ga.attn_forward(q, q, q, out=out, heads=1, headDim=128, window=-3)
    t.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 7.0)
