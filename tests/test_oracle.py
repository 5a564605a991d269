"""Pins for the attention oracle: each test ties it to something other than itself.

The pages print no worked example, so the pins are the page's own rules
written out by hand (golden files), the catalogue's primitive ops composed,
a library routine (torch's CPU f64 scaled_dot_product_attention), closed
forms at chosen numbers, and invariants that the definition implies. A
plausible slip in the oracle (a dropped term, a wrong sign, a wrong index or
stride, a transposed operand) fails at least one of them.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import alibi as oracle_alibi
import workloads
from tests import page_ops as ops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def _rand(shape, seed, std=1.0):
    return workloads.normal(shape, seed, 0, std)


# --------------------------------------------------------------------------
# Golden: the page's window rule, evaluated by hand (tests/golden).
# --------------------------------------------------------------------------

def _uniform_weights_row(causal, S, pos, window):
    """With q = 0 every visible key gets the same weight; v = identity reads them off."""
    q = np.zeros((1, 4), np.float32)
    k = _rand((S, 4), 1)
    v = np.eye(S, dtype=np.float32)
    out = oracle.attention(q, k, v, heads=1, headDim=4, vHeadDim=S, causal=bool(causal),
                           posOffset=pos, window=window)
    return out[0]


def test_golden_window_visibility():
    cases = 0
    for line in _golden_lines("window_visibility.txt"):
        lhs, rhs = line.split(":")
        causal, S, pos, window = (int(x) for x in lhs.split())
        visible = [int(x) for x in rhs.split()]
        row = _uniform_weights_row(causal, S, pos, window)
        want = np.zeros(S)
        want[visible] = 1.0 / len(visible)
        np.testing.assert_allclose(row, want, rtol=0, atol=1e-15, err_msg=line)
        cases += 1
    assert cases >= 10


def test_golden_window_empty_rows_are_zero():
    # Reading for rows with no visible key (parity unpinned; see the fixture).
    for line in _golden_lines("window_visibility_empty.txt"):
        causal, S, pos, window = (int(x) for x in line.split(":")[0].split())
        row = _uniform_weights_row(causal, S, pos, window)
        assert np.all(row == 0.0), line


# --------------------------------------------------------------------------
# Golden: ALiBi slopes as the ALiBi paper lists them.
# --------------------------------------------------------------------------

def test_golden_alibi_slopes():
    for line in _golden_lines("alibi_slopes.txt"):
        lhs, rhs = line.split(":")
        H = int(lhs)
        want = [2.0 ** float(e) for e in rhs.split()]
        assert len(want) == H
        np.testing.assert_allclose(oracle_alibi.bloom_slopes(H), want, rtol=1e-15, atol=0)
        np.testing.assert_allclose(oracle_alibi.mpt_slopes(H, 8.0), want, rtol=1e-15, atol=0)


@pytest.mark.parametrize("H", list(range(1, 65)))
def test_alibi_bloom_equals_mpt_at_bias_max_8(H):
    # Two different published constructions that coincide when alibi_bias_max is 8
    # (for a power of two H trivially; otherwise through MPT's even/odd reordering).
    np.testing.assert_allclose(oracle_alibi.bloom_slopes(H), oracle_alibi.mpt_slopes(H, 8.0),
                               rtol=1e-15, atol=0)


def test_alibi_mpt_other_bias_max_closed_form():
    # alibi_bias_max 16 with 8 heads: 2^(-16 i / 8) = 4^-i.
    np.testing.assert_allclose(oracle_alibi.mpt_slopes(8, 16.0), [4.0 ** -i for i in range(1, 9)],
                               rtol=1e-15)
    # 12 heads at b = 8: the 8 slopes 2^-1..2^-8, then 2^-0.5, 2^-1.5, 2^-2.5, 2^-3.5.
    want = [2.0 ** -i for i in range(1, 9)] + [2.0 ** -(j + 0.5) for j in range(4)]
    np.testing.assert_allclose(oracle_alibi.mpt_slopes(12, 8.0), want, rtol=1e-15)


def test_alibi_precedence():
    # alibiSlopes > alibiMax > alibi (reading where the page is silent).
    r = oracle.resolve(1, 1, heads=2, headDim=4, alibi=True, alibiMax=16.0, alibiSlopes=[0.5, 0.25])
    assert r["slopes"] == [0.5, 0.25]
    r = oracle.resolve(1, 1, heads=2, headDim=4, alibi=True, alibiMax=16.0)
    assert r["slopes"] == [oracle.f32(2.0 ** -8), oracle.f32(2.0 ** -16)]
    r = oracle.resolve(1, 1, heads=2, headDim=4, alibi=True)
    assert r["slopes"] == [2.0 ** -4, 2.0 ** -8]


# --------------------------------------------------------------------------
# Closed forms at chosen numbers.
# --------------------------------------------------------------------------

def _sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z))


def test_closed_form_two_keys_default_scale():
    # headDim 4: the default scale is 1/2, and q.k1 = 2, so the scores are 0 and 1.
    q = np.ones((1, 4), np.float32)
    k = np.array([[0, 0, 0, 0], [0.5, 0.5, 0.5, 0.5]], np.float32)
    v = np.array([[0.0], [1.0]], np.float32)
    out = oracle.attention(q, k, v, heads=1, headDim=4, vHeadDim=1, causal=False)
    assert out[0, 0] == pytest.approx(_sigmoid(1.0), abs=1e-15)


def test_closed_form_scale_override():
    q = np.ones((1, 4), np.float32)
    k = np.array([[0, 0, 0, 0], [0.5, 0.5, 0.5, 0.5]], np.float32)
    v = np.array([[0.0], [1.0]], np.float32)
    out = oracle.attention(q, k, v, heads=1, headDim=4, vHeadDim=1, causal=False, scale=1.5)
    assert out[0, 0] == pytest.approx(_sigmoid(3.0), abs=1e-15)


def test_closed_form_softcap_saturates_and_bias_masks_after_it():
    # Scores 1000 and 2000 capped at 10 both become ~10: equal weights, mean of v.
    q = np.ones((1, 1), np.float32)
    k = np.array([[1000.0], [2000.0]], np.float32)
    v = np.array([[2.0], [4.0]], np.float32)
    out = oracle.attention(q, k, v, heads=1, headDim=1, causal=False, scale=1.0, softcap=10.0)
    assert out[0, 0] == pytest.approx(3.0, abs=1e-12)
    # Without the cap, the larger score takes all the weight.
    out = oracle.attention(q, k, v, heads=1, headDim=1, causal=False, scale=1.0)
    assert out[0, 0] == pytest.approx(4.0, abs=1e-12)
    # A -1e9 bias still masks when softcap is on: it is added after the cap
    # (the catalogue puts softcap ahead of masking; the bias is how a
    # caller masks). Were it capped, the key would keep weight e^-20.
    bias = np.array([[0.0, -1e9]], np.float32)
    out = oracle.attention(q, k, v, bias, heads=1, headDim=1, causal=False, scale=1.0, softcap=10.0)
    assert out[0, 0] == 2.0


def test_closed_form_softcap_value():
    # One visible key pair with scores 0 and s: weight of the second is sigmoid(c tanh(s/c)).
    c, s = 2.0, 3.0
    q = np.ones((1, 1), np.float32)
    k = np.array([[0.0], [s]], np.float32)
    v = np.array([[0.0], [1.0]], np.float32)
    out = oracle.attention(q, k, v, heads=1, headDim=1, causal=False, scale=1.0, softcap=c)
    assert out[0, 0] == pytest.approx(_sigmoid(c * math.tanh(s / c)), abs=1e-15)


def test_closed_form_alibi_causal_geometric():
    # q = 0, one head, slope ln 2 (as its f32 value m): causal weights fall by e^-m per step back.
    S = 7
    m = np.float32(math.log(2.0))
    q = np.zeros((1, 2), np.float32)
    k = _rand((S, 2), 3)
    v = np.eye(S, dtype=np.float32)
    w = oracle.attention(q, k, v, heads=1, headDim=2, vHeadDim=S, posOffset=S - 1,
                         alibiSlopes=[float(m)])[0]
    ratios = w[:-1] / w[1:]
    np.testing.assert_allclose(ratios, math.exp(-float(m)), rtol=1e-13)
    geo = sum(math.exp(-float(m) * d) for d in range(S))
    assert w[-1] == pytest.approx(1.0 / geo, rel=1e-13)


def test_closed_form_alibi_noncausal_symmetric():
    # Non-causal: the penalty is symmetric in |pos - s| (reading; the page is silent).
    S, pos = 9, 4
    q = np.zeros((1, 2), np.float32)
    k = _rand((S, 2), 3)
    v = np.eye(S, dtype=np.float32)
    w = oracle.attention(q, k, v, heads=1, headDim=2, vHeadDim=S, causal=False, posOffset=pos,
                         alibiSlopes=[0.5])[0]
    np.testing.assert_allclose(w[:pos][::-1], w[pos + 1:], rtol=1e-14)
    np.testing.assert_allclose(w[:-1][pos:] / w[1:][pos:], math.exp(0.5), rtol=1e-13)


def test_closed_form_gqa_head_mapping():
    # Contiguous groups: with H=6, G=3, heads 0,1 read KV head 0, heads 2,3 head 1, 4,5 head 2.
    H, G, S = 6, 3, 5
    q = _rand((2, H * 2), 4)
    k = _rand((S, G * 2), 5)
    v = np.concatenate([np.full((S, 1), g + 1.0, np.float32) for g in range(G)], axis=1)
    out = oracle.attention(q, k, v, heads=H, kvHeads=G, headDim=2, vHeadDim=1, causal=False)
    np.testing.assert_allclose(out, np.tile([1, 1, 2, 2, 3, 3], (2, 1)), atol=1e-14)


@pytest.mark.parametrize("layout", ["TS", "HTS"])
def test_closed_form_bias_indexing(layout):
    # Every key is masked but one chosen per (head, row); the output is that key's v row.
    H, T, S = 3, 4, 6
    q = _rand((T, H * 2), 6)
    k = _rand((S, 2), 7)
    v = np.eye(S, dtype=np.float32)
    pick = np.array([[(3 * h + 5 * t + 1) % S for t in range(T)] for h in range(H)])
    if layout == "TS":
        pick[:] = pick[0]
        bias = np.full((T, S), -1e9, np.float32)
        for t in range(T):
            bias[t, pick[0, t]] = 0.0
    else:
        bias = np.full((H, T, S), -1e9, np.float32)
        for h in range(H):
            for t in range(T):
                bias[h, t, pick[h, t]] = 0.0
    out = oracle.attention(q, k, v, bias, heads=H, kvHeads=1, headDim=2, vHeadDim=S, causal=False)
    for h in range(H):
        for t in range(T):
            want = np.zeros(S)
            want[pick[h, t]] = 1.0
            np.testing.assert_array_equal(out[t, h * S:(h + 1) * S], want)


def test_closed_form_posoffset_rows():
    # Two query rows at positions 3 and 4 see keys 0..3 and 0..4.
    S = 6
    q = np.zeros((2, 2), np.float32)
    k = _rand((S, 2), 8)
    v = np.eye(S, dtype=np.float32)
    out = oracle.attention(q, k, v, heads=1, headDim=2, vHeadDim=S, posOffset=3)
    np.testing.assert_allclose(out[0], [.25, .25, .25, .25, 0, 0], atol=1e-15)
    np.testing.assert_allclose(out[1], [.2, .2, .2, .2, .2, 0], atol=1e-15)


# --------------------------------------------------------------------------
# Invariants the definition implies.
# --------------------------------------------------------------------------

def test_rows_sum_to_one():
    T, S, H, G, D = 5, 9, 4, 2, 8
    q, k = _rand((T, H * D), 10, 3.0), _rand((S, G * D), 11, 3.0)
    v = np.ones((S, G * 3), np.float32)
    bias = workloads.masked_bias((H, T, S), 12, 0.3)
    bias[:, :, 0] = 0.0  # key 0 stays unmasked on every row
    out = oracle.attention(q, k, v, bias, heads=H, kvHeads=G, headDim=D, vHeadDim=3,
                           posOffset=S - T, softcap=5.0, alibi=True, window=6)
    np.testing.assert_allclose(out, 1.0, atol=1e-14)


def test_single_key_returns_v():
    H, G, D, Dv = 4, 2, 8, 5
    q, k, v = _rand((1, H * D), 13), _rand((1, G * D), 14), _rand((1, G * Dv), 15)
    out = oracle.attention(q, k, v, heads=H, kvHeads=G, headDim=D, vHeadDim=Dv, softcap=3.0,
                           alibi=True)
    want = np.concatenate([v[0, (h * G // H) * Dv:(h * G // H + 1) * Dv] for h in range(H)])
    np.testing.assert_array_equal(out[0], want.astype(np.float64))


def test_zero_query_is_mean_of_visible_v():
    T, S, H, G, D, Dv = 4, 7, 4, 2, 3, 2
    q = np.zeros((T, H * D), np.float32)
    k, v = _rand((S, G * D), 16), _rand((S, G * Dv), 17)
    out = oracle.attention(q, k, v, heads=H, kvHeads=G, headDim=D, vHeadDim=Dv, posOffset=2)
    vv = v.astype(np.float64)
    for t in range(T):
        for h in range(H):
            g = h * G // H
            want = vv[:2 + t + 1, g * Dv:(g + 1) * Dv].mean(axis=0)
            np.testing.assert_allclose(out[t, h * Dv:(h + 1) * Dv], want, atol=1e-15)


def test_gqa_equals_repeated_kv_heads():
    T, S, H, G, D, Dv = 5, 8, 8, 2, 4, 3
    q, k, v = _rand((T, H * D), 18), _rand((S, G * D), 19), _rand((S, G * Dv), 20)
    rep = H // G
    k_rep = np.concatenate([k[:, (h // rep) * D:(h // rep + 1) * D] for h in range(H)], axis=1)
    v_rep = np.concatenate([v[:, (h // rep) * Dv:(h // rep + 1) * Dv] for h in range(H)], axis=1)
    kw = dict(heads=H, headDim=D, vHeadDim=Dv, posOffset=3, alibi=True, softcap=4.0)
    a = oracle.attention(q, k, v, kvHeads=G, **kw)
    b = oracle.attention(q, k_rep, v_rep, kvHeads=H, **kw)
    np.testing.assert_array_equal(a, b)


def test_wide_window_equals_causal_and_full():
    T, S, H, D = 4, 9, 2, 4
    q, k, v = _rand((T, H * D), 21), _rand((S, D), 22), _rand((S, D), 23)
    kw = dict(heads=H, kvHeads=1, headDim=D, posOffset=5)
    np.testing.assert_array_equal(oracle.attention(q, k, v, window=5 + T, **kw),
                                  oracle.attention(q, k, v, **kw))
    np.testing.assert_array_equal(oracle.attention(q, k, v, causal=False, window=S + 5 + T, **kw),
                                  oracle.attention(q, k, v, causal=False, **kw))


def test_bias_mask_equals_causal():
    T, S, H, G, D = 5, 9, 4, 2, 4
    q, k, v = _rand((T, H * D), 24), _rand((S, G * D), 25), _rand((S, G * D), 26)
    P0 = 3
    bias = np.zeros((T, S), np.float32)
    for t in range(T):
        bias[t, P0 + t + 1:] = -1e9
    kw = dict(heads=H, kvHeads=G, headDim=D, posOffset=P0)
    np.testing.assert_array_equal(oracle.attention(q, k, v, bias, causal=False, **kw),
                                  oracle.attention(q, k, v, causal=True, **kw))


def test_chunked_and_decode_rows_equal_full_prefill_rows():
    S, H, G, D = 12, 4, 2, 8
    q, k, v = _rand((S, H * D), 27), _rand((S, G * D), 28), _rand((S, G * D), 29)
    kw = dict(heads=H, kvHeads=G, headDim=D, window=7, softcap=6.0, alibi=True)
    full = oracle.attention(q, k, v, **kw)
    chunk = oracle.attention(q[8:], k, v, posOffset=8, **kw)
    np.testing.assert_array_equal(chunk, full[8:])
    dec = oracle.attention(q[5:6], k, v, posOffset=5, **kw)
    np.testing.assert_array_equal(dec, full[5:6])
    sub = oracle.attention(q, k, v, rows=[11, 0, 6], **kw)
    np.testing.assert_array_equal(sub, full[[11, 0, 6]])


def test_alibi_equals_bias_with_same_penalty():
    # Power-of-two slopes times small integer distances are exact in f32,
    # so the bias path sees exactly the same numbers.
    T, S, H, D = 3, 10, 8, 4
    q, k, v = _rand((T, H * D), 30), _rand((S, D), 31), _rand((S, D), 32)
    for causal in (True, False):
        P0 = 6
        slopes = oracle_alibi.bloom_slopes(H)
        bias = np.zeros((H, T, S), np.float32)
        for h in range(H):
            for t in range(T):
                for s in range(S):
                    bias[h, t, s] = -slopes[h] * abs(P0 + t - s)
        kw = dict(heads=H, kvHeads=1, headDim=D, posOffset=P0, causal=causal)
        np.testing.assert_array_equal(oracle.attention(q, k, v, alibi=True, **kw),
                                      oracle.attention(q, k, v, bias, **kw))


def mpt_full_alibi(H: int, S: int, alibi_bias_max: float = 8.0) -> np.ndarray:
    """MPT's bidirectional ("full") ALiBi bias for an S x S block, built the
    way that model builds it: a row vector of key positions 1-S .. 0, minus
    the same positions as a column (the query positions), made non-positive
    by taking minus its absolute value, then scaled per head by MPT's slopes
    (2^(-i b / n) over the next power of two n >= H, even-numbered first).
    Returns [H, S, S] f32."""
    pos = np.arange(1 - S, 1, dtype=np.float64)
    diff = pos[None, :] - pos[:, None]                       # key minus query
    dist = -np.abs(diff)
    n = 1 << (H - 1).bit_length()
    m = np.array([2.0 ** (-(i + 1) * alibi_bias_max / n) for i in range(n)])
    if n != H:
        m = np.concatenate([m[1::2], m[0::2]])[:H]
    return (dist[None, :, :] * m[:, None, None]).astype(np.float32)


@pytest.mark.parametrize("H, S", [(8, 12), (6, 9), (16, 5)])
def test_noncausal_alibi_is_mpt_full_bias(H, S):
    # The non-causal ALiBi reading (-slope * |pos - s|) is MPT's bidirectional
    # bias: the oracle's alibiMax path must equal the same call with MPT's own
    # construction passed as the bias input. With 8 or 6 heads the slopes are
    # powers of two, so slope times distance is exact in f32 and the two agree
    # bit for bit; 16 heads have slopes 2^(-i/2), where the bias input holds
    # the f32 rounding of each product (the oracle rounds the slope once),
    # a difference far below the bar. Also with a window.
    D = 4
    q, k, v = _rand((S, H * D), 40 + H), _rand((S, 2 * D), 41), _rand((S, 2 * D), 42)
    bias = mpt_full_alibi(H, S, 8.0)
    for extra in ({}, dict(window=3)):
        kw = dict(heads=H, kvHeads=2 if H % 2 == 0 else 1, headDim=D, causal=False, **extra)
        if kw["kvHeads"] == 1:
            kv = (k[:, :D].copy(), v[:, :D].copy())
        else:
            kv = (k, v)
        got = oracle.attention(q, *kv, alibiMax=8.0, **kw)
        want = oracle.attention(q, *kv, bias, **kw)
        if H == 16:
            np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)
        else:
            np.testing.assert_array_equal(got, want)


def test_noncausal_alibi_mpt_bias_on_a_shifted_block():
    # Rows at positions P0..P0+T-1 of a longer key range: the rows of MPT's
    # S x S construction at those positions (its positions are shifted by a
    # constant, which the differences do not see).
    H, S, T, P0, D = 8, 14, 5, 6, 4
    q, k, v = _rand((T, H * D), 45), _rand((S, D), 46), _rand((S, D), 47)
    bias = np.ascontiguousarray(mpt_full_alibi(H, S)[:, P0:P0 + T, :])
    kw = dict(heads=H, kvHeads=1, headDim=D, causal=False, posOffset=P0)
    np.testing.assert_array_equal(oracle.attention(q, k, v, alibi=True, **kw),
                                  oracle.attention(q, k, v, bias, **kw))


def test_alibi_relative_equals_bloom_absolute_when_causal():
    # BLOOM adds +m*s; on causal rows -m*|pos - s| differs by the row constant -m*pos.
    T, S, H, D = 4, 11, 8, 4
    q, k, v = _rand((T, H * D), 33), _rand((S, D), 34), _rand((S, D), 35)
    slopes = oracle_alibi.bloom_slopes(H)
    absolute = np.zeros((H, T, S), np.float32)
    for h in range(H):
        absolute[h, :, :] = np.float32(slopes[h]) * np.arange(S, dtype=np.float32)
    kw = dict(heads=H, kvHeads=1, headDim=D, posOffset=S - T)
    np.testing.assert_allclose(oracle.attention(q, k, v, alibi=True, **kw),
                               oracle.attention(q, k, v, absolute, **kw), rtol=0, atol=1e-12)


def test_huge_softcap_is_no_softcap():
    T, S, H, D = 3, 6, 2, 4
    q, k, v = _rand((T, H * D), 36), _rand((S, D), 37), _rand((S, D), 38)
    kw = dict(heads=H, kvHeads=1, headDim=D, posOffset=3)
    np.testing.assert_allclose(oracle.attention(q, k, v, softcap=1e30, **kw),
                               oracle.attention(q, k, v, **kw), rtol=0, atol=1e-12)


def test_threads_do_not_change_result():
    T, S, H, G, D = 6, 10, 4, 2, 8
    q, k, v = _rand((T, H * D), 39), _rand((S, G * D), 40), _rand((S, G * D), 41)
    kw = dict(heads=H, kvHeads=G, headDim=D, posOffset=4, alibi=True)
    np.testing.assert_array_equal(oracle.attention(q, k, v, threads=1, **kw),
                                  oracle.attention(q, k, v, threads=7, **kw))


# --------------------------------------------------------------------------
# The catalogue's primitives composed (T = S, posOffset 0, no window).
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("use_softcap", [False, True])
@pytest.mark.parametrize("bias_layout", [None, "TS", "HTS"])
def test_composition_of_catalogue_ops(causal, use_softcap, bias_layout):
    T = S = 7
    H, G, D, Dv = 4, 2, 6, 5
    sigma = 0.3
    q, k, v = _rand((T, H * D), 42, 2.0), _rand((S, G * D), 43, 2.0), _rand((S, G * Dv), 44)
    bias = None
    if bias_layout == "TS":
        bias = workloads.masked_bias((T, S), 45, 0.2)
    elif bias_layout == "HTS":
        bias = workloads.masked_bias((H, T, S), 45, 0.2)
    if bias is not None:
        bias[..., 0] = 0.0  # keep one visible key on every row
    c = 1.5 if use_softcap else None
    got = oracle.attention(q, k, v, bias, heads=H, kvHeads=G, headDim=D, vHeadDim=Dv,
                           causal=causal, scale=sigma, softcap=c)
    for h in range(H):
        g = h * G // H
        qh = ops.slice_(q, h * D, D, axis=-1)
        kg = ops.slice_(k, g * D, D, axis=-1)
        vg = ops.slice_(v, g * Dv, Dv, axis=-1)
        x = ops.matmul(qh, kg, transB=True)
        x = ops.scale(x, np.float32(sigma))
        if c is not None:
            x = ops.softcap(x, c)
        if bias is not None:
            x = ops.add(x, bias if bias.ndim == 2 else bias[h])
        if causal:
            x = ops.causal_mask(x)
        want = ops.matmul(ops.softmax(x), vg)
        np.testing.assert_allclose(got[:, h * Dv:(h + 1) * Dv], want, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# A library routine: torch's CPU f64 scaled_dot_product_attention.
# --------------------------------------------------------------------------

def _sdpa_reference(q, k, v, bias, H, G, D, Dv, causal, P0, sigma, window, slopes):
    T, S = q.shape[0], k.shape[0]
    qt = torch.from_numpy(q.astype(np.float64)).view(T, H, D).transpose(0, 1)
    kt = torch.from_numpy(k.astype(np.float64)).view(S, G, D).transpose(0, 1)
    vt = torch.from_numpy(v.astype(np.float64)).view(S, G, Dv).transpose(0, 1)
    kt = kt.repeat_interleave(H // G, dim=0).contiguous()
    vt = vt.repeat_interleave(H // G, dim=0).contiguous()
    pos = P0 + torch.arange(T, dtype=torch.int64)[:, None]
    s = torch.arange(S, dtype=torch.int64)[None, :]
    if causal:
        vis = s <= pos
        if window:
            vis &= s > pos - window
    else:
        vis = torch.ones(T, S, dtype=torch.bool)
        if window:
            vis &= (pos - s).abs() <= window
    mask = torch.zeros(H, T, S, dtype=torch.float64)
    if slopes is not None:
        mask -= torch.tensor(slopes, dtype=torch.float64)[:, None, None] * (pos - s).abs().double()
    if bias is not None:
        mask += torch.from_numpy(bias.astype(np.float64))
    mask = mask.masked_fill(~vis, float("-inf"))
    out = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None],
                                                           attn_mask=mask[None], scale=sigma)
    return out[0].transpose(0, 1).reshape(T, H * Dv).numpy()


def _sdpa_cases():
    rng = np.random.default_rng(1234)
    cases = []
    for i in range(40):
        H = int(rng.choice([1, 2, 4, 6, 8]))
        G = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
        D = int(rng.choice([1, 3, 8, 16]))
        Dv = int(rng.choice([D, 2, 5]))
        S = int(rng.integers(1, 13))
        causal = bool(rng.integers(0, 2))
        T = int(rng.integers(1, S + 1)) if causal else int(rng.integers(1, 10))
        P0 = int(rng.integers(0, S - T + 1)) if causal else int(rng.integers(0, S + 3))
        window = int(rng.choice([0, 0, 1, 3, 6]))
        if not causal and window:
            window = max(window, P0 + T)  # keep a visible key on every row
        alibi = int(rng.integers(0, 3))
        bias = [None, "TS", "HTS"][int(rng.integers(0, 3))]
        scale = None if rng.integers(0, 2) else float(rng.uniform(0.05, 1.0))
        cases.append((i, H, G, D, Dv, T, S, causal, P0, window, alibi, bias, scale))
    return cases


@pytest.mark.parametrize("case", _sdpa_cases(), ids=lambda c: f"case{c[0]}")
def test_matches_torch_sdpa_f64(case):
    i, H, G, D, Dv, T, S, causal, P0, window, alibi, bias_layout, scale = case
    q, k, v = _rand((T, H * D), 100 + i, 1.5), _rand((S, G * D), 200 + i, 1.5), _rand((S, G * Dv), 300 + i)
    bias = None
    if bias_layout == "TS":
        bias = workloads.normal((T, S), 400 + i, 3, 1.0)
    elif bias_layout == "HTS":
        bias = workloads.normal((H, T, S), 400 + i, 3, 1.0)
    params = dict(heads=H, kvHeads=G, headDim=D, vHeadDim=Dv, causal=causal, posOffset=P0,
                  window=window)
    if scale is not None:
        params["scale"] = scale
    if alibi == 1:
        params["alibi"] = True
    elif alibi == 2:
        params["alibiSlopes"] = [0.1 * (h + 1) for h in range(H)]
    r = oracle.resolve(T, S, **params)
    got = oracle.attention(q, k, v, bias, **params)
    want = _sdpa_reference(q, k, v, bias, H, G, D, Dv, causal, P0, r["scale"], window, r["slopes"])
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


def test_llama_decode_shape_matches_torch_sdpa_on_sampled_heads():
    # The decode workload's real shapes, with a shortened cache to keep this quick.
    w = workloads.LLAMA_DECODE.replace(S=2048, posOffset=2047)
    q, k, v, _ = w.tensors()
    got = oracle.attention(q, k, v, **w.params())
    r = oracle.resolve(w.T, w.S, **w.params())
    want = _sdpa_reference(q, k, v, None, 32, 8, 128, 128, True, 2047, r["scale"], 0, None)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# Parameter handling and cache_write.
# --------------------------------------------------------------------------

def test_defaults_resolve():
    r = oracle.resolve(3, 5, heads=8, headDim=128)
    assert (r["G"], r["Dv"], r["causal"], r["P0"], r["softcap"], r["window"], r["slopes"]) == \
        (8, 128, True, 0, 0.0, 0, None)
    assert r["scale"] == oracle.f32(1 / math.sqrt(128))
    r = oracle.resolve(1, 1, heads=16, headDim=192, vHeadDim=128)
    assert r["scale"] == oracle.f32(1 / math.sqrt(192))  # headDim, not vHeadDim


@pytest.mark.parametrize("bad", [dict(kvHeads=3), dict(posOffset=-1), dict(softcap=-1.0),
                                 dict(window=-2), dict(alibiSlopes=[1.0])])
def test_invalid_params_refused(bad):
    with pytest.raises(ValueError):
        oracle.resolve(2, 2, heads=4, headDim=8, **bad)


def test_cache_write_copies_rows_exactly():
    cache = workloads.normal((10, 6), 1, 1)
    before = cache.copy()
    vals = workloads.normal((3, 6), 1, 2)
    out = oracle.cache_write(cache, vals, 4)
    assert out is cache
    assert np.array_equal(cache[4:7].view(np.uint32), vals.view(np.uint32))
    assert np.array_equal(cache[:4], before[:4]) and np.array_equal(cache[7:], before[7:])
    with pytest.raises(ValueError):
        oracle.cache_write(cache, vals, 8)


# --------------------------------------------------------------------------
# Attention sinks (the IR schema's `sinks` beside `window`; the reading is
# StreamingLLM's kept initial tokens: keys s < sinks stay visible).
# --------------------------------------------------------------------------

def _uniform_weights_row_sinks(causal, S, pos, window, sinks):
    q = np.zeros((1, 4), np.float32)
    k = _rand((S, 4), 1)
    v = np.eye(S, dtype=np.float32)
    return oracle.attention(q, k, v, heads=1, headDim=4, vHeadDim=S, causal=bool(causal),
                            posOffset=pos, window=window, sinks=sinks)[0]


def test_golden_sink_visibility():
    cases = 0
    for line in _golden_lines("sink_visibility.txt"):
        lhs, rhs = line.split(":")
        causal, S, pos, window, sinks = (int(x) for x in lhs.split())
        visible = [int(x) for x in rhs.split()]
        row = _uniform_weights_row_sinks(causal, S, pos, window, sinks)
        want = np.zeros(S)
        want[visible] = 1.0 / len(visible)
        np.testing.assert_allclose(row, want, rtol=0, atol=1e-15, err_msg=line)
        cases += 1
    assert cases >= 10


def test_closed_form_one_sink_and_a_one_key_window():
    # Causal row at position 5 with window 1 and one sink sees keys 0 and 5
    # only; scores 0.5 * q.k are 0 and 1 (headDim 4, default scale 1/2).
    q = np.ones((1, 4), np.float32)
    k = np.full((6, 4), 9.0, np.float32)              # hidden keys would dominate if seen
    k[0] = 0.0
    k[5] = 0.5
    v = np.arange(6, dtype=np.float32)[:, None] * 10.0
    out = oracle.attention(q, k, v, heads=1, headDim=4, vHeadDim=1, posOffset=5, window=1, sinks=1)
    w5 = _sigmoid(1.0)
    assert out[0, 0] == pytest.approx(w5 * 50.0 + (1 - w5) * 0.0, abs=1e-12)


def test_sinks_zero_or_without_window_change_nothing():
    T, S, H, G, D = 6, 20, 4, 2, 8
    q, k, v = _rand((T, H * D), 61), _rand((S, G * D), 62), _rand((S, G * D), 63)
    for causal in (True, False):
        kw = dict(heads=H, kvHeads=G, headDim=D, posOffset=12, causal=causal)
        np.testing.assert_array_equal(oracle.attention(q, k, v, window=4, sinks=0, **kw),
                                      oracle.attention(q, k, v, window=4, **kw))
        np.testing.assert_array_equal(oracle.attention(q, k, v, sinks=5, **kw),
                                      oracle.attention(q, k, v, **kw))


def test_all_keys_sinks_is_plain_causal():
    T, S, H, D = 5, 16, 2, 4
    q, k, v = _rand((T, H * D), 64), _rand((S, D), 65), _rand((S, D), 66)
    kw = dict(heads=H, kvHeads=1, headDim=D, posOffset=11)
    np.testing.assert_array_equal(oracle.attention(q, k, v, window=2, sinks=S, **kw),
                                  oracle.attention(q, k, v, **kw))


@pytest.mark.parametrize("causal", [True, False])
def test_sinks_equal_a_bias_mask(causal):
    # A -1e9 bias on every key outside (sinks U window) and no window gives the
    # same result bit for bit (exp underflows to exactly 0).
    T, S, H, G, D, P0, w, n = 6, 30, 4, 2, 8, 20, 5, 3
    q, k, v = _rand((T, H * D), 67), _rand((S, G * D), 68), _rand((S, G * D), 69)
    bias = np.zeros((T, S), np.float32)
    for t in range(T):
        pos = P0 + t
        for s in range(S):
            inwin = (pos - w < s <= pos) if causal else abs(pos - s) <= w
            if not (inwin or s < n):
                bias[t, s] = -1e9
    kw = dict(heads=H, kvHeads=G, headDim=D, posOffset=P0, causal=causal)
    np.testing.assert_array_equal(oracle.attention(q, k, v, bias, **kw),
                                  oracle.attention(q, k, v, window=w, sinks=n, **kw))


def _sdpa_with_sinks(q, k, v, H, G, D, causal, P0, sigma, window, sinks):
    T, S = q.shape[0], k.shape[0]
    qt = torch.from_numpy(q.astype(np.float64)).view(T, H, D).transpose(0, 1)
    kt = torch.from_numpy(k.astype(np.float64)).view(S, G, D).transpose(0, 1).repeat_interleave(H // G, 0)
    vt = torch.from_numpy(v.astype(np.float64)).view(S, G, D).transpose(0, 1).repeat_interleave(H // G, 0)
    pos = P0 + torch.arange(T)[:, None]
    s = torch.arange(S)[None, :]
    win = ((s <= pos) & (s > pos - window)) if causal else ((pos - s).abs() <= window)
    sink = (s < sinks) & ((s <= pos) if causal else torch.ones_like(win))
    mask = torch.zeros(T, S, dtype=torch.float64).masked_fill(~(win | sink), float("-inf"))
    out = torch.nn.functional.scaled_dot_product_attention(qt.contiguous()[None], kt.contiguous()[None],
                                                           vt.contiguous()[None], attn_mask=mask,
                                                           scale=sigma)
    return out[0].transpose(0, 1).reshape(T, H * D).numpy()


@pytest.mark.parametrize("causal, T, S, P0, window, sinks", [
    (True, 7, 40, 33, 4, 4), (True, 16, 16, 0, 3, 2), (True, 1, 64, 63, 8, 1),
    (False, 9, 30, 10, 2, 5), (False, 4, 12, 0, 1, 3)])
def test_sinks_match_torch_sdpa_f64(causal, T, S, P0, window, sinks):
    H, G, D = 4, 2, 8
    q, k, v = _rand((T, H * D), 70 + T, 1.5), _rand((S, G * D), 71 + S, 1.5), _rand((S, G * D), 72)
    got = oracle.attention(q, k, v, heads=H, kvHeads=G, headDim=D, posOffset=P0, causal=causal,
                           window=window, sinks=sinks)
    sigma = oracle.f32(1 / math.sqrt(D))   # the scale enters as an f32 number
    want = _sdpa_with_sinks(q, k, v, H, G, D, causal, P0, sigma, window, sinks)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_negative_sinks_refused():
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 4), np.float32), np.zeros((2, 4), np.float32),
                         np.zeros((2, 4), np.float32), heads=1, headDim=4, window=1, sinks=-1)
