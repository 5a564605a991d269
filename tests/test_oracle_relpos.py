"""Pins for the two relative-position score terms of the attention oracle.

The IR schema page lists `position_bias` {weight, buckets} and `relative_kv`
{key, value, max_distance} on its attention op without a rule. The oracle
reads them as T5's bucketed relative position bias and Shaw et al.'s relative
position representations. The pins tie that to: hand-evaluated bucket rows
(tests/golden), T5's bucket function written from its published definition
(log-spaced buckets past half the bucket count), the bias input of the same
op fed the equivalent numbers, keys and values materialized per query row and
handed to the pinned core or to torch's f64 SDPA, and closed forms.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, stream=0, std=1.0):
    return workloads.normal(shape, seed, stream, std)


# --------------------------------------------------------------------------
# position_bias
# --------------------------------------------------------------------------

def test_golden_bucket_rows():
    cases = 0
    with open(os.path.join(GOLDEN, "position_bias_buckets.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            th, bi, pos, rows = (x.strip() for x in line.split("|"))
            th = [int(x) for x in th.split()]
            bi, pos = int(bi), int(pos)
            want = [int(x) for x in rows.split()]
            S, n = len(want), len(th)
            nrows = 2 * n if bi else n
            # q = 0: every visible key scores its bias only; bias_r = log(r + 1)
            # gives key s the weight (row(s) + 1) / sum, read off by v = identity.
            weight = np.log(np.arange(1, nrows + 1, dtype=np.float64))[:, None].astype(np.float32)
            q = np.zeros((1, 4), np.float32)
            out = oracle.attention(q, _rand((S, 4), 1), np.eye(S, dtype=np.float32), heads=1, headDim=4,
                                   vHeadDim=S, causal=False, posOffset=pos,
                                   position_bias=dict(weight=weight, buckets=th, bidirectional=bool(bi)))
            w = np.exp(weight[want, 0].astype(np.float64))
            np.testing.assert_allclose(out[0], w / w.sum(), rtol=1e-12, atol=1e-15, err_msg=line)
            cases += 1
    assert cases >= 5


def t5_bucket(rel, bidirectional, num_buckets, max_distance):
    """T5's relative-position bucket of rel = key position - query position:
    half the buckets (per direction when bidirectional) are exact distances,
    the rest log-spaced up to max_distance, the last one open-ended."""
    ret = 0
    n = -rel
    if bidirectional:
        num_buckets //= 2
        if rel > 0:
            ret += num_buckets
        n = abs(rel)
    else:
        n = max(n, 0)
    max_exact = num_buckets // 2
    if n < max_exact:
        return ret + n
    large = max_exact + int(math.log(n / max_exact) / math.log(max_distance / max_exact)
                            * (num_buckets - max_exact))
    return ret + min(large, num_buckets - 1)


def t5_thresholds(num_buckets, max_distance, bidirectional, upto=4096):
    """The first distance of each bucket (keys at or before the query)."""
    per_side = num_buckets // 2 if bidirectional else num_buckets
    th = {}
    for d in range(upto):
        b = t5_bucket(-d, bidirectional, num_buckets, max_distance)
        th.setdefault(b, d)
    assert sorted(th) == list(range(per_side))
    return [th[b] for b in range(per_side)]


@pytest.mark.parametrize("bidirectional", [False, True])
def test_t5_bucket_function_equals_thresholds(bidirectional):
    # Thresholds taken from T5's bucket function reproduce it as a bias input.
    H, T, S, P0 = 3, 5, 300, 200
    nb, md = 32, 128
    th = t5_thresholds(nb, md, bidirectional)
    per = len(th)
    weight = _rand((2 * per if bidirectional else per, H), 5, 3)
    bias = np.empty((H, T, S), np.float32)
    for t in range(T):
        for s in range(S):
            b = t5_bucket(s - (P0 + t), bidirectional, nb, md)
            bias[:, t, s] = weight[b]
    q, k, v = _rand((T, H * 8), 1), _rand((S, H * 8), 2), _rand((S, H * 8), 3)
    kw = dict(heads=H, headDim=8, posOffset=P0, causal=not bidirectional)
    got = oracle.attention(q, k, v, position_bias=dict(weight=weight, buckets=th, bidirectional=bidirectional),
                           **kw)
    want = oracle.attention(q, k, v, bias, **kw)
    np.testing.assert_array_equal(got, want)


def test_closed_form_two_keys():
    # q = 0, keys at distances 1 and 0 in buckets 1 and 0 with biases a and b.
    a, b = 0.75, -0.5
    q = np.zeros((1, 2), np.float32)
    v = np.array([[1.0], [0.0]], np.float32)
    out = oracle.attention(q, _rand((2, 2), 4), v, heads=1, headDim=2, vHeadDim=1, posOffset=1,
                           position_bias=dict(weight=np.array([[b], [a]], np.float32), buckets=[0, 1]))
    assert out[0, 0] == pytest.approx(1.0 / (1.0 + math.exp(b - a)), abs=1e-15)


def test_position_bias_constant_shift_per_head_cancels():
    H, T, S = 2, 4, 40
    th = [0, 1, 2, 4, 8, 16]
    weight = _rand((len(th), H), 7)
    q, k, v = _rand((T, H * 8), 1), _rand((S, H * 8), 2), _rand((S, H * 8), 3)
    kw = dict(heads=H, headDim=8, posOffset=S - T)
    a = oracle.attention(q, k, v, position_bias=dict(weight=weight, buckets=th), **kw)
    shifted = weight + np.array([[1.5, -2.0]], np.float32)
    b = oracle.attention(q, k, v, position_bias=dict(weight=shifted, buckets=th), **kw)
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-6)
    # ... while a change to one bucket's bias changes the output.
    bumped = weight.copy()
    bumped[2, 0] += 2.0
    c = oracle.attention(q, k, v, position_bias=dict(weight=bumped, buckets=th), **kw)
    assert np.abs(c[:, :8] - a[:, :8]).max() > 1e-3 and np.array_equal(c[:, 8:], a[:, 8:])


@pytest.mark.parametrize("bad", [dict(buckets=[1, 2]), dict(buckets=[0, 2, 2]), dict(buckets=[0, 3, 1]),
                                 dict(weight=np.zeros((2, 2), np.float32))])
def test_position_bias_refused(bad):
    pb = dict(weight=np.zeros((3, 2), np.float32), buckets=[0, 1, 2])
    pb.update(bad)
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 8), np.float32), np.zeros((2, 8), np.float32),
                         np.zeros((2, 8), np.float32), heads=2, headDim=4, position_bias=pb)


# --------------------------------------------------------------------------
# relative_kv
# --------------------------------------------------------------------------

def _rel_row(s, pos, m):
    return min(max(s - pos, -m), m) + m


CASES = [dict(causal=True, m=3, P0=10, with_v=True), dict(causal=False, m=2, P0=0, with_v=True),
         dict(causal=True, m=0, P0=4, with_v=False), dict(causal=False, m=20, P0=5, with_v=True, window=3)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_relative_kv_equals_per_row_materialized_keys(case):
    c = CASES[case]
    H, G, D, Dv, T, S = 4, 2, 8, 6, 4, 17
    m = c["m"]
    q, k, v = _rand((T, H * D), 1), _rand((S, G * D), 2), _rand((S, G * Dv), 3)
    rk = _rand((2 * m + 1, D), 4, 1)
    rv = _rand((2 * m + 1, Dv), 5, 2) if c["with_v"] else None
    kw = dict(heads=H, kvHeads=G, headDim=D, vHeadDim=Dv, causal=c["causal"], window=c.get("window"))
    got = oracle.attention(q, k, v, posOffset=c["P0"],
                           relative_kv=dict(key=rk, value=rv, max_distance=m), **kw)
    for t in range(T):
        pos = c["P0"] + t
        idx = [_rel_row(s, pos, m) for s in range(S)]
        k2 = (k.reshape(S, G, D).astype(np.float64) + rk[idx][:, None, :]).astype(np.float32).reshape(S, G * D)
        v2 = v.reshape(S, G, Dv).astype(np.float64)
        if rv is not None:
            v2 = v2 + rv[idx][:, None, :]
        v2 = v2.astype(np.float32).reshape(S, G * Dv)
        want = oracle.attention(q[t:t + 1], k2, v2, posOffset=pos, **kw)
        # Materializing rounds k + rel_k and v + rel_v to f32 once.
        np.testing.assert_allclose(got[t], want[0], rtol=5e-6, atol=5e-6)


def test_relative_kv_matches_torch_sdpa_f64():
    H, D, T, S, m, P0 = 2, 8, 3, 12, 2, 9
    q, k, v = _rand((T, H * D), 1), _rand((S, H * D), 2), _rand((S, H * D), 3)
    rk, rv = _rand((2 * m + 1, D), 4, 1), _rand((2 * m + 1, D), 5, 2)
    got = oracle.attention(q, k, v, heads=H, headDim=D, posOffset=P0,
                           relative_kv=dict(key=rk, value=rv, max_distance=m))
    for t in range(T):
        pos = P0 + t
        idx = [_rel_row(s, pos, m) for s in range(S)]
        vis = np.arange(S) <= pos
        for h in range(H):
            kk = k[:, h * D:(h + 1) * D].astype(np.float64) + rk[idx]
            vv = v[:, h * D:(h + 1) * D].astype(np.float64) + rv[idx]
            mask = torch.from_numpy(np.where(vis, 0.0, -np.inf)[None, :])
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[t:t + 1, h * D:(h + 1) * D].astype(np.float64)), torch.from_numpy(kk),
                torch.from_numpy(vv), attn_mask=mask, scale=float(np.float32(1 / math.sqrt(D))))
            np.testing.assert_allclose(got[t, h * D:(h + 1) * D], o.numpy()[0], rtol=1e-12, atol=1e-12)


def test_relative_kv_distance_zero_closed_form():
    # max_distance 0: every key takes row 0, so the key term is the same for
    # all keys of a row (no effect) and the value term adds rel_v[0].
    H, D, T, S = 2, 8, 3, 10
    q, k, v = _rand((T, H * D), 1), _rand((S, H * D), 2), _rand((S, H * D), 3)
    rk, rv = _rand((1, D), 4, 1), _rand((1, D), 5, 2)
    got = oracle.attention(q, k, v, heads=H, headDim=D, posOffset=7,
                           relative_kv=dict(key=rk, value=rv, max_distance=0))
    plain = oracle.attention(q, k, v, heads=H, headDim=D, posOffset=7)
    np.testing.assert_allclose(got, plain + np.tile(rv[0].astype(np.float64), H), rtol=1e-12, atol=1e-12)


def test_zero_relative_tables_are_plain_attention():
    H, D, T, S, m = 2, 8, 3, 10, 4
    q, k, v = _rand((T, H * D), 1), _rand((S, H * D), 2), _rand((S, H * D), 3)
    z = np.zeros((2 * m + 1, D), np.float32)
    got = oracle.attention(q, k, v, heads=H, headDim=D, posOffset=7,
                           relative_kv=dict(key=z, value=z, max_distance=m))
    np.testing.assert_array_equal(got, oracle.attention(q, k, v, heads=H, headDim=D, posOffset=7))


@pytest.mark.parametrize("bad", [dict(max_distance=-1), dict(key=np.zeros((4, 8), np.float32)),
                                 dict(value=np.zeros((5, 3), np.float32))])
def test_relative_kv_refused(bad):
    rk = dict(key=np.zeros((5, 8), np.float32), value=None, max_distance=2)
    rk.update(bad)
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 8), np.float32), np.zeros((2, 8), np.float32),
                         np.zeros((2, 8), np.float32), heads=1, headDim=8, relative_kv=rk)
