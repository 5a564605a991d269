"""Latent (MLA) attention on the GPU (attn_mla_forward) against the f64 oracle.

The library evaluates the absorbed form (q through k_b first, the softmax
over the latent rows, v_b last); the oracle materializes every head's keys
and values. Same bar as attention: |gpu - ref| <= 1e-4 + 1e-4 |ref|.
"""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
from oracle import mla
import workloads
from tests.parity import assert_close, dev, torch

pytestmark = pytest.mark.gpu


def _run(w, tensors=None, **kw):
    q, state, k_b, v_b = tensors if tensors is not None else w.tensors()
    out = ga.attn_mla_forward(dev(q), dev(state), dev(k_b), dev(v_b), **w.params(), **kw)
    torch().cuda.synchronize()
    return out.cpu().numpy()


def _check(w, tensors=None, what=""):
    tensors = tensors if tensors is not None else w.tensors()
    got = _run(w, tensors)
    ref = mla.mla_attention(*tensors, **w.params())
    assert_close(got, ref, what or w.name)
    return got


def _wl(**kw):
    base = dict(name="mla", T=1, S=300, heads=16, kv_rank=512, qk_nope=128, qk_rope=64, v_head_dim=128)
    base.update(kw)
    if "posOffset" not in kw and base.get("causal", True) is not False:
        base["posOffset"] = base["S"] - base["T"]
    return workloads.MlaWorkload(**base)


@pytest.mark.parametrize("R, P", [(512, 64), (256, 64)])
@pytest.mark.parametrize("T, H, S", [(1, 16, 300), (1, 3, 77), (2, 16, 1000), (5, 7, 129), (33, 4, 64),
                                     (1, 128, 513)])
def test_mla_matrix_core_shapes(R, P, T, H, S):
    w = _wl(T=T, S=S, heads=H, kv_rank=R, qk_rope=P, seed=T + H)
    assert ga.attn_mla_plan(w.T, w.S, **w.params())["tile_q"] == 16
    _check(w, what=f"R={R} T={T} H={H} S={S}")


@pytest.mark.parametrize("S", [1, 15, 16, 17, 31, 33])
def test_mla_ragged_key_counts(S):
    _check(_wl(S=S, heads=5, seed=S), what=f"S={S}")


@pytest.mark.parametrize("N, Dv", [(64, 32), (192, 100), (16, 7)])
def test_mla_head_widths(N, Dv):
    _check(_wl(qk_nope=N, v_head_dim=Dv, heads=4, S=200), what=f"qk_nope={N} v_head_dim={Dv}")


@pytest.mark.parametrize("R, P, N", [(48, 16, 24), (96, 0, 32), (512, 32, 128)])
def test_mla_generic_shapes(R, P, N):
    w = _wl(kv_rank=R, qk_rope=P, qk_nope=N, heads=3, T=3, S=90, v_head_dim=24)
    assert ga.attn_mla_plan(w.T, w.S, **w.params())["tile_q"] == 1
    _check(w, what=f"generic R={R} P={P}")


@pytest.mark.parametrize("kw", [dict(causal=False), dict(causal=False, window=40),
                                dict(window=100), dict(window=64, sinks=4), dict(window=3, sinks=1),
                                dict(scale=0.05), dict(T=6, posOffset=700, S=706),
                                dict(T=4, causal=False, window=5, sinks=2, posOffset=50)])
def test_mla_features(kw):
    w = _wl(S=kw.get("S", 900), heads=16, **{k: v for k, v in kw.items() if k != "S"})
    _check(w, what=str(kw))
    try:
        ga.attn_set_option("mla_generic", 1)
        _check(w, what=f"generic {kw}")
    finally:
        ga.attn_set_option("mla_generic", 0)


@pytest.mark.parametrize("splits", [1, 2, 7, 40])
def test_mla_forced_splits(splits):
    # Window 900 at positions 1998-1999: keys 1099..1999 (901 rows) split
    # into chunks of a multiple of 16 keys, then the sink split for keys 0..7.
    w = _wl(S=2000, T=2, heads=16, window=900, sinks=8)
    try:
        ga.attn_set_option("mla_splits", splits)
        chunk = -(-(-(-901 // splits)) // 16) * 16
        assert ga.attn_mla_plan(w.T, w.S, **w.params())["splits"] == -(-901 // chunk) + 1
        _check(w, what=f"splits={splits}")
    finally:
        ga.attn_set_option("mla_splits", 0)


@pytest.mark.parametrize("out", [16, 32])
@pytest.mark.parametrize("kw", [dict(S=2000, T=2, heads=16, window=900, sinks=8), dict(S=700, T=1, heads=40),
                                dict(S=1500, T=1, heads=16, kv_rank=256, v_head_dim=96)])
def test_mla_combine_widths(out, kw):
    # The per-output merge: workgroups of 16 or 32 output channels (v_head_dim
    # 96 leaves a partial last group at 32).
    w = _wl(**kw)
    try:
        ga.attn_set_option("mla_slices", -1)
        ga.attn_set_option("mla_combine_out", out)
        assert ga.attn_mla_plan(w.T, w.S, **w.params())["slices"] == 0
        _check(w, what=f"combine_out={out} {kw}")
    finally:
        ga.attn_set_option("mla_combine_out", 0)
        ga.attn_set_option("mla_slices", 0)


def test_mla_never_reads_past_the_position_or_the_gap():
    # Causal decode over a cache of 4096 rows at position 2999: rows past it
    # and rows between the sinks and the window hold NaN.
    w = _wl(S=4096, T=1, posOffset=2999, window=1000, sinks=4)
    q, state, k_b, v_b = w.tensors()
    poisoned = state.copy()
    poisoned[3000:] = np.nan
    poisoned[4:2000] = np.nan
    got = _run(w, (q, poisoned, k_b, v_b))
    ref = mla.mla_attention(q, state, k_b, v_b, **w.params())
    assert_close(got, ref, "poisoned state")


def test_mla_rows_with_no_key_are_zero():
    w = _wl(S=10, T=2, posOffset=100, causal=False, window=5)  # every key is out of reach
    assert ga.attn_mla_plan(w.T, w.S, **w.params())["path"] == "zero"
    assert np.all(_run(w) == 0.0)
    w0 = _wl(S=0, T=1, posOffset=0)
    q, _, k_b, v_b = w0.tensors()
    empty = torch().empty((0, w0.kv_rank + w0.qk_rope), device="cuda")
    out = ga.attn_mla_forward(dev(q), empty, dev(k_b), dev(v_b), **w0.params())
    assert np.all(out.cpu().numpy() == 0.0)


def test_mla_is_deterministic():
    w = _wl(S=3000, heads=16)
    a = _run(w)
    b = _run(w)
    assert np.array_equal(a, b)


def test_mla_v2_lite_decode_full_size():
    w = workloads.MLA_DECODE
    _check(w)


def test_mla_v3_decode_full_size_sampled_heads():
    # 128 heads over a 32768-row state; heads are independent, so the oracle
    # computes a sample of them one at a time.
    w = workloads.MLA_DECODE_V3
    q, state, k_b, v_b = w.tensors()
    got = _run(w, (q, state, k_b, v_b))
    N, P, Dv = w.qk_nope, w.qk_rope, w.v_head_dim
    for h in (0, 1, 17, 64, 127):
        one = w.replace(heads=1)
        qh = np.ascontiguousarray(q[:, h * (N + P):(h + 1) * (N + P)])
        ref = mla.mla_attention(qh, state, k_b[h:h + 1], v_b[h:h + 1], **one.params())
        assert_close(got[:, h * Dv:(h + 1) * Dv], ref, f"v3 head {h}")


@pytest.fixture
def slice_merge():
    ga.attn_set_option("mla_slices", 1)  # also the automatic choice for these shapes
    yield
    ga.attn_set_option("mla_slices", 0)


@pytest.mark.parametrize("kw", [dict(T=1, S=300, heads=16), dict(T=2, S=1000, heads=16), dict(T=5, S=129, heads=7),
                                dict(T=33, S=64, heads=4), dict(T=1, S=513, heads=128),
                                dict(T=1, S=300, heads=3, kv_rank=256), dict(T=3, S=700, heads=5, v_head_dim=100),
                                dict(T=2, S=90, heads=4, v_head_dim=7, qk_nope=16),
                                dict(T=1, S=200, heads=4, v_head_dim=256, qk_nope=192),
                                dict(S=2000, T=2, heads=16, window=900, sinks=8), dict(S=900, causal=False, window=40),
                                dict(S=900, T=4, causal=False, window=5, sinks=2, posOffset=50),
                                dict(S=17, T=1, heads=5), dict(S=1, T=1, heads=2)])
def test_mla_slice_merge(kw, slice_merge):
    # The merge by latent slices: each slice workgroup projects its share,
    # the row's last one adds the shares.
    w = _wl(**kw)
    plan = ga.attn_mla_plan(w.T, w.S, **w.params())
    assert plan["slices"] == w.kv_rank // 64, plan
    _check(w, what=f"slices {kw}")


def test_mla_slice_merge_empty_rows(slice_merge):
    # Window 1 at positions S-1 and S: the second row sees only key S, past
    # the state, so its output is exactly zero while the first row's is not.
    w = _wl(S=50, T=2, heads=4, window=1, posOffset=49)
    got = _check(w, what="slices, one empty row")
    assert np.all(got[1] == 0.0) and np.any(got[0] != 0.0)


@pytest.mark.parametrize("splits", [1, 3, 250, 1000])
def test_mla_slice_merge_split_counts(splits, slice_merge):
    # Split counts past one batch of accumulator loads per thread (8 x 16).
    w = _wl(S=16000, T=1, heads=4)
    try:
        ga.attn_set_option("mla_splits", splits)
        assert ga.attn_mla_plan(w.T, w.S, **w.params())["splits"] == splits
        _check(w, what=f"slices, splits={splits}")
    finally:
        ga.attn_set_option("mla_splits", 0)


def test_mla_slice_merge_repeated_calls(slice_merge):
    # Each call's counters start from zero: back-to-back calls with one
    # workspace, a larger then a smaller problem, give the same bits as fresh ones.
    big, small = _wl(S=3000, T=2, heads=16), _wl(S=500, T=1, heads=4)
    tb, ts = big.tensors(), small.tensors()
    ws = torch().empty(max(ga.attn_mla_workspace_size(big.T, big.S, **big.params()),
                           ga.attn_mla_workspace_size(small.T, small.S, **small.params())),
                       dtype=torch().uint8, device="cuda")
    def run(w, t):
        o = ga.attn_mla_forward(dev(t[0]), dev(t[1]), dev(t[2]), dev(t[3]), workspace=ws, **w.params())
        torch().cuda.synchronize()
        return o.cpu().numpy()
    first = [run(big, tb), run(small, ts)]
    for _ in range(3):
        assert np.array_equal(run(big, tb), first[0])
        assert np.array_equal(run(small, ts), first[1])
    assert_close(first[0], mla.mla_attention(*tb, **big.params()), "slices, repeated big")
    assert_close(first[1], mla.mla_attention(*ts, **small.params()), "slices, repeated small")


def test_mla_slice_merge_full_size(slice_merge):
    _check(workloads.MLA_DECODE, what="slices, V2-Lite-shaped")
    w = workloads.MLA_DECODE_V3
    q, state, k_b, v_b = w.tensors()
    got = _run(w, (q, state, k_b, v_b))
    N, P, Dv = w.qk_nope, w.qk_rope, w.v_head_dim
    for h in (0, 5, 63, 127):
        one = w.replace(heads=1)
        qh = np.ascontiguousarray(q[:, h * (N + P):(h + 1) * (N + P)])
        ref = mla.mla_attention(qh, state, k_b[h:h + 1], v_b[h:h + 1], **one.params())
        assert_close(got[:, h * Dv:(h + 1) * Dv], ref, f"slices, v3 head {h}")
