"""80- and 96-wide heads (Phi-2, StableLM-3B; Phi-3-mini, GPT-NeoX-20B) on the
decode kernel, whose 16-lane row layout leaves part of the second float4 group
of each row empty, against the oracle on the GPU."""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import workloads
from tests.parity import compare, dev, run_library, torch
from tests.test_gpu_append import _append
from tests.test_gpu_relpos import _check_pb, _check_rkv, _pb

pytestmark = pytest.mark.gpu

WIDTHS = [80, 96]


def _wl(D, **kw):
    base = dict(name=f"D={D} decode", T=1, S=1000, heads=8, kvHeads=2, headDim=D, posOffset=999, seed=D)
    base.update(kw)
    return workloads.Workload(**base)


def _check(w, what=None, expect_path="decode", out=None):
    q, k, v, bias = w.tensors()
    plan = ga.attn_plan(w.T, w.S, bias_kind={None: 0, "TS": 1, "HTS": 2}[w.bias], **w.params())
    assert plan["path"] == expect_path, plan
    return compare(q, k, v, bias, w.params(), what=what or w.name, out=out)


@pytest.mark.parametrize("D", WIDTHS)
@pytest.mark.parametrize("H, G, T", [(8, 2, 1), (16, 16, 1), (8, 4, 1), (4, 1, 1), (8, 8, 2), (6, 3, 1), (8, 8, 3),
                                     (16, 2, 1), (32, 32, 1), (12, 4, 2)])
def test_width_decode_shapes(D, H, G, T):
    S = 777
    _check(_wl(D, T=T, S=S, heads=H, kvHeads=G, posOffset=S - T, seed=D + H + T), what=f"D={D} H={H} G={G} T={T}")


@pytest.mark.parametrize("D", WIDTHS)
@pytest.mark.parametrize("feature", [
    dict(window=100), dict(window=64, sinks=4), dict(softcap=5.0, std=3.0), dict(alibi=True),
    dict(bias="TS", bias_mask_prob=0.1), dict(bias="HTS", bias_mask_prob=0.3), dict(causal=False),
    dict(causal=False, window=50, posOffset=500),
    dict(softcap=20.0, window=300, alibi=True, bias="HTS", bias_mask_prob=0.1, std=2.0),
])
def test_width_decode_features(D, feature):
    _check(_wl(D, **feature), what=f"D={D} {feature}")


@pytest.mark.parametrize("opt, val", [("decode_splits", 1), ("decode_splits", 5), ("decode_splits", 64),
                                      ("decode_block", 64), ("decode_depth", 2), ("decode_depth", 3)])
def test_width_decode_plan_options(opt, val):
    w = _wl(80, S=6000, posOffset=5999, heads=16, kvHeads=4)
    try:
        ga.attn_set_option(opt, val)
        _check(w, what=f"D=80 {opt}={val}")
    finally:
        ga.attn_set_option(opt, 0)


@pytest.mark.parametrize("D", WIDTHS)
def test_width_decode_never_reads_past_the_position(D):
    # Rows past the query's position hold NaN: they must not reach the output.
    w = _wl(D, S=2048, posOffset=1499)
    q, k, v, _ = w.tensors()
    kp, vp = k.copy(), v.copy()
    kp[1500:] = np.nan
    vp[1500:] = np.nan
    got = run_library(q, kp, vp, None, w.params()).cpu().numpy()
    want = run_library(q, k, v, None, w.params()).cpu().numpy()
    np.testing.assert_array_equal(got, want)
    assert np.isfinite(got).all()


@pytest.mark.parametrize("D", WIDTHS)
def test_width_decode_output_guard_bands_untouched(D):
    # Each lane stores only the channels inside its row: the neighbours of
    # the output stay as they were.
    t = torch()
    w = _wl(D, heads=16, kvHeads=4)
    n, pad = w.T * 16 * D, 64
    big = t.full((n + 2 * pad,), float("nan"), dtype=t.float32, device="cuda")
    out = big[pad:pad + n].view(w.T, 16 * D)
    _check(w, what=f"D={D} guarded out", out=out)
    b = big.cpu().numpy()
    assert np.isnan(b[:pad]).all() and np.isnan(b[-pad:]).all()


@pytest.mark.parametrize("D", WIDTHS)
@pytest.mark.parametrize("kw", [dict(T=1, S=3000, heads=32, kvHeads=8), dict(T=3, S=900, heads=4, kvHeads=2),
                                dict(T=1, S=2049, heads=8, kvHeads=8, alibi=True, bias="TS", bias_mask_prob=0.1)])
def test_width_fused_append(D, kw):
    # The appended rows are read from their buffers and stored into the
    # caches by the decode kernel itself: every cache bit is checked, and no
    # lane may write past its row.
    w = workloads.Workload(name=f"D={D} append", headDim=D, posOffset=kw["S"] - kw["T"], seed=D + kw["S"], **kw)
    assert _append(w, w.T, w.posOffset, poison_past=w.posOffset + w.T) == 0


@pytest.mark.parametrize("D", WIDTHS)
@pytest.mark.parametrize("m", [0, 16, 200])
def test_width_relative_kv_decode(D, m):
    w = workloads.Workload("rkv decode", T=1, S=3000, heads=8, kvHeads=2, headDim=D, posOffset=2999, seed=D + m)
    _check_rkv(w, m, True, ("decode", "generic"))


@pytest.mark.parametrize("D", WIDTHS)
def test_width_position_bias_decode(D):
    w = workloads.Workload("pb decode", T=1, S=3000, heads=8, kvHeads=4, headDim=D, posOffset=2999, seed=D)
    th, weight = _pb(8)
    _check_pb(w, th, weight, False, ("decode", "generic"))


# --------------------------------------------------------------------------
# 80- and 96-wide heads on the 32x32x2 prefill kernel: 96-wide tiles (80-wide
# rows padded with zero columns), three output floats per lane and k-step.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("D", WIDTHS)
@pytest.mark.parametrize("kw", [dict(T=300, S=300, heads=8, kvHeads=2, posOffset=0),
                                dict(T=77, S=1077, heads=4, kvHeads=4, posOffset=1000),
                                dict(T=130, S=130, heads=32, kvHeads=32, posOffset=0),
                                dict(T=64, S=200, heads=16, kvHeads=1, posOffset=136),
                                dict(T=1, S=700, heads=64, kvHeads=2, posOffset=699)])
def test_width_prefill_shapes(D, kw):
    w = _wl(D, name=f"D={D} prefill", **kw)
    assert ga.attn_plan(w.T, w.S, **w.params())["variant"] == 32
    _check(w, what=f"D={D} {kw}", expect_path="prefill")


@pytest.mark.parametrize("D", WIDTHS)
@pytest.mark.parametrize("feature", [
    dict(window=100), dict(window=64, sinks=4), dict(softcap=5.0, std=3.0), dict(alibi=True),
    dict(bias="TS", bias_mask_prob=0.1), dict(bias="HTS", bias_mask_prob=0.3), dict(causal=False),
    dict(causal=False, window=50),
])
def test_width_prefill_features(D, feature):
    w = _wl(D, name=f"D={D} prefill feature", T=200, S=260, heads=8, kvHeads=2, posOffset=60, **feature)
    _check(w, what=f"D={D} {feature}", expect_path="prefill")


@pytest.mark.parametrize("D", WIDTHS)
@pytest.mark.parametrize("splits", [2, 5])
def test_width_prefill_key_splits(D, splits):
    w = _wl(D, name=f"D={D} chunked", T=100, S=2100, heads=8, kvHeads=2, posOffset=2000)
    try:
        ga.attn_set_option("prefill_splits", splits)
        assert ga.attn_plan(w.T, w.S, **w.params())["splits"] == splits
        _check(w, what=f"D={D} splits={splits}", expect_path="prefill")
    finally:
        ga.attn_set_option("prefill_splits", 0)


@pytest.mark.parametrize("D", WIDTHS)
def test_width_prefill_output_guard_bands_untouched(D):
    # Lanes whose columns lie past the row (the padding of 80-wide rows) store
    # nothing: the neighbours of the output stay as they were.
    t = torch()
    w = _wl(D, name=f"D={D} prefill guarded", T=96, S=96, heads=4, kvHeads=2, posOffset=0)
    n, pad = w.T * 4 * D, 64
    big = t.full((n + 2 * pad,), float("nan"), dtype=t.float32, device="cuda")
    out = big[pad:pad + n].view(w.T, 4 * D)
    _check(w, what=f"D={D} prefill guarded out", expect_path="prefill", out=out)
    b = big.cpu().numpy()
    assert np.isnan(b[:pad]).all() and np.isnan(b[-pad:]).all()


@pytest.mark.parametrize("D", WIDTHS)
def test_width_prefill_with_rotary_q(D):
    # q turned as it is loaded (half-split pairs over the whole width).
    import oracle
    from tests.parity import assert_close
    w = _wl(D, name=f"D={D} rope prefill", T=150, S=150, heads=8, kvHeads=2, posOffset=0)
    q, k, v, _ = w.tensors()
    qr = dict(base=10000.0)
    roped = oracle.rope(q, headDim=D, offset=0, **qr).astype(np.float32)
    ref = oracle.attention(roped, k, v, None, **w.params())
    out = ga.attn_forward(dev(q), dev(k), dev(v), **w.params(), q_rope=dict(qr))
    torch().cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, f"D={D} rope prefill")


@pytest.mark.parametrize("D", WIDTHS)
@pytest.mark.parametrize("m", [0, 16, 200])
@pytest.mark.parametrize("causal", [True, False])
def test_width_relative_kv_prefill(D, m, causal):
    w = workloads.Workload(f"D={D} rkv prefill", T=150, S=230 if causal else 200, heads=8, kvHeads=2, headDim=D,
                           posOffset=80 if causal else 30, causal=causal, seed=D + m)
    _check_rkv(w, m, True, (None, "generic"), seed=m)


@pytest.mark.parametrize("D", WIDTHS)
def test_width_prefill_full_size_sampled(D):
    # A Phi-shaped causal prefill: 32 heads over 2048 rows.
    from tests.parity import sample_rows
    w = _wl(D, name=f"D={D} 2048", T=2048, S=2048, heads=32, kvHeads=32, posOffset=0)
    q, k, v, _ = w.tensors()
    assert ga.attn_plan(w.T, w.S, **w.params())["path"] == "prefill"
    compare(q, k, v, None, w.params(), rows=sample_rows(w.T, seed=D), what=f"D={D} 2048 sampled")


@pytest.mark.parametrize("D", WIDTHS)
def test_width_prefill_key_splits_many_rows(D):
    # Many output rows and few key-range parts: the merge takes one thread per
    # output float4 (combine_few) at these widths.
    from tests.parity import sample_rows
    w = _wl(D, name=f"D={D} split many rows", T=1024, S=3072, heads=32, kvHeads=8, posOffset=2048)
    q, k, v, _ = w.tensors()
    try:
        ga.attn_set_option("prefill_splits", 3)
        assert ga.attn_plan(w.T, w.S, **w.params())["splits"] == 3
        compare(q, k, v, None, w.params(), rows=sample_rows(w.T, seed=D + 1), what=f"D={D} combine_few")
    finally:
        ga.attn_set_option("prefill_splits", 0)


@pytest.mark.parametrize("D", WIDTHS)
def test_width_fused_append_with_rotary_q(D):
    # The decode kernel turns q through LDS: lanes past the row's width take zeros.
    import oracle
    from tests.parity import assert_close
    w = _wl(D, name=f"D={D} rope decode", S=640, posOffset=639, heads=8, kvHeads=2)
    qr = dict(base=10000.0)
    q, k, v, _ = w.tensors()
    roped = oracle.rope(q, headDim=D, offset=w.posOffset, **qr).astype(np.float32)
    ref = oracle.attention(roped, k, v, None, **w.params())
    kc, vc = dev(k), dev(v)
    kc[-1] = float("nan")
    vc[-1] = float("nan")
    out = ga.attn_forward_append(dev(q), kc, vc, dev(k[-1:]), dev(v[-1:]), w.S - 1, q_rope=dict(qr), **w.params())
    torch().cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, f"D={D} rotary q decode")
    np.testing.assert_array_equal(kc.cpu().numpy().view(np.uint32), k.view(np.uint32))
