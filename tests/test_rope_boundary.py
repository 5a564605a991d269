"""The rope entry points' host side, checked on the CPU (no device calls).

The library resolves the op's parameters into an f32 inverse-frequency table
and attention factor; these must equal the oracle's bit for bit (both compute
each value in double and round once), because at position p a one-ulp change
of a frequency moves the angle by p ulps. Bad arguments are refused by name
before any launch.
"""

import ctypes

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import oracle
from gqa_scaled_dot_amd import _lib

LONG = list(np.linspace(1.0, 8.0, 32))
SHORT = list(np.linspace(1.0, 2.0, 32))

TABLE_CASES = [
    ("default", dict(headDim=128), 1),
    ("default-odd-base", dict(headDim=64, base=12345.678), 1),
    ("partial", dict(headDim=128, rotaryDim=32, base=500000.0), 1),
    ("two-channels", dict(headDim=10, rotaryDim=2), 1),
    ("rotary-256", dict(headDim=256, base=1e6), 1),
    ("linear", dict(headDim=64, scaling=dict(rope_type="linear", factor=4.0)), 1),
    ("linear-type-key", dict(headDim=64, scaling=dict(type="linear", factor=2.5)), 1),
    ("llama3", dict(headDim=128, base=500000.0,
                    scaling=dict(rope_type="llama3", factor=8.0, low_freq_factor=1.0,
                                 high_freq_factor=4.0, original_max_position_embeddings=8192)), 1),
    ("llama3-defaults", dict(headDim=64, base=10000.0,
                             scaling=dict(rope_type="llama3", factor=4.0,
                                          original_max_position_embeddings=2048)), 1),
    ("yarn", dict(headDim=64, scaling=dict(rope_type="yarn", factor=4.0,
                                           original_max_position_embeddings=4096)), 1),
    ("yarn-mscale", dict(headDim=64, scaling=dict(rope_type="yarn", factor=40.0, beta_fast=32,
                                                  beta_slow=1, mscale=1.0, mscale_all_dim=0.707,
                                                  original_max_position_embeddings=4096)), 1),
    ("yarn-untruncated", dict(headDim=128, base=1e6,
                              scaling=dict(rope_type="yarn", factor=4.0, truncate=False,
                                           original_max_position_embeddings=32768)), 1),
    ("yarn-own-factor", dict(headDim=64, scaling=dict(rope_type="yarn", factor=4.0,
                                                      original_max_position_embeddings=4096,
                                                      attention_factor=1.25)), 1),
    ("dynamic-short", dict(headDim=64, scaling=dict(rope_type="dynamic", factor=2.0,
                                                    max_position_embeddings=4096)), 100),
    ("dynamic-long", dict(headDim=64, offset=9000,
                          scaling=dict(rope_type="dynamic", factor=2.0,
                                       original_max_position_embeddings=4096)), 7),
    ("longrope-short", dict(headDim=64, scaling=dict(rope_type="longrope", short_factor=SHORT,
                                                     long_factor=LONG,
                                                     original_max_position_embeddings=4096,
                                                     max_position_embeddings=131072)), 10),
    ("longrope-long", dict(headDim=64, offset=4090,
                           scaling=dict(rope_type="longrope", short_factor=SHORT, long_factor=LONG,
                                        original_max_position_embeddings=4096, factor=32.0)), 10),
    ("explicit", dict(headDim=16, invFreq=[0.5 ** i for i in range(8)], attentionFactor=0.9), 1),
    ("explicit-wins", dict(headDim=16, invFreq=list(np.linspace(2.0, 0.1, 8)),
                           scaling=dict(rope_type="linear", factor=3.0)), 1),
]


@pytest.mark.parametrize("name, kw, rows", TABLE_CASES, ids=[c[0] for c in TABLE_CASES])
def test_library_table_is_the_oracles_bit_for_bit(name, kw, rows):
    got, af = ga.attn_rope_table(rows=rows, **kw)
    rd = kw.get("rotaryDim") or kw["headDim"]
    want, waf = oracle.rope_table(rd, base=kw.get("base"), scaling=kw.get("scaling"),
                                  invFreq=kw.get("invFreq"), attentionFactor=kw.get("attentionFactor"),
                                  seq_len=(kw.get("offset") or 0) + rows)
    assert got.dtype == np.float32 and got.shape == want.shape
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.float32(af) == np.float32(waf)


def test_rope_params_init_defaults():
    r = _lib.AttnRopeParams()
    ctypes.memset(ctypes.byref(r), 0xFF, ctypes.sizeof(r))
    _lib.lib().attn_rope_params_init(ctypes.byref(r))
    assert (r.head_dim, r.rotary_dim, r.offset, r.interleaved, r.scaling) == (0, 0, 0, 0, 0)
    assert r.base == 0.0 and not r.inv_freq and r.has_attention_factor == 0 and r.truncate == 1
    assert not r.short_factor and not r.long_factor and r.scaling_attention_factor == 0.0


@pytest.mark.parametrize("kw, code, word", [
    (dict(headDim=0), 1, "headDim"),
    (dict(headDim=64, rotaryDim=63), 1, "rotaryDim"),
    (dict(headDim=64, rotaryDim=66), 1, "rotaryDim"),
    (dict(headDim=512), 2, "rotaryDim"),
    (dict(headDim=64, offset=-3), 1, "offset"),
    (dict(headDim=64, offset=2**31), 1, "offset"),
    (dict(headDim=64, base=-1.0), 1, "base"),
    (dict(headDim=64, attentionFactor=float("inf")), 1, "attentionFactor"),
    (dict(headDim=64, scaling=dict(rope_type="linear")), 1, "factor"),
    (dict(headDim=64, scaling=dict(rope_type="llama3", factor=8.0)), 1, "original"),
    (dict(headDim=64, scaling=dict(rope_type="llama3", factor=8.0, low_freq_factor=4.0,
                                   high_freq_factor=1.0, original_max_position_embeddings=8192)),
     1, "llama3"),
    (dict(headDim=64, scaling=dict(rope_type="yarn", factor=4.0)), 1, "original"),
    (dict(headDim=64, scaling=dict(rope_type="longrope", original_max_position_embeddings=4096)),
     1, "longrope"),
    (dict(headDim=64, scaling=dict(rope_type="longrope", short_factor=SHORT, long_factor=LONG,
                                   original_max_position_embeddings=4096)), 1, "longrope"),
    (dict(headDim=64, scaling=dict(rope_type="dynamic", factor=2.0)), 1, "dynamic"),
    (dict(headDim=2, scaling=dict(rope_type="dynamic", factor=2.0, max_position_embeddings=4)),
     1, "rotaryDim"),
    (dict(headDim=4, invFreq=[1.0, float("nan")]), 1, "invFreq"),
])
def test_bad_rope_params_are_refused_by_name(kw, code, word):
    with pytest.raises(ga.AttnError) as e:
        ga.attn_rope_table(**kw)
    assert e.value.code == code and word in e.value.message, e.value.message


def test_binding_checks_list_lengths_and_scaling_names():
    with pytest.raises(ga.AttnError) as e:
        ga.attn_rope_table(headDim=64, invFreq=[1.0] * 31)
    assert "invFreq" in e.value.message
    with pytest.raises(ga.AttnError) as e:
        ga.attn_rope_table(headDim=64, scaling=dict(rope_type="ntk-magic", factor=2.0))
    assert e.value.code == 2 and "scaling" in e.value.message
    with pytest.raises(ga.AttnError):
        ga.attn_rope_table(headDim=64, scaling=dict(rope_type="longrope", short_factor=[1.0] * 3,
                                                    long_factor=LONG,
                                                    original_max_position_embeddings=4096))


def _rope_raw(r, T, width, x, out):
    return _lib.lib().attn_rope(ctypes.byref(r), T, width, x, out, None)


def test_rope_refuses_before_launch():
    A = 1 << 32
    r, keep = ga.make_rope_params(headDim=64)
    assert _rope_raw(r, 4, 100, A, 2 * A) == 1 and "headDim" in ga.attn_last_error()
    assert _rope_raw(r, -1, 128, A, 2 * A) == 1 and "rows" in ga.attn_last_error()
    assert _rope_raw(r, 4, 128, None, 2 * A) == 1 and "x" in ga.attn_last_error()
    assert _rope_raw(r, 4, 128, A, A + 64) == 1 and "overlap" in ga.attn_last_error()
    assert _rope_raw(r, 0, 128, None, None) == 0  # T = 0: no-op
    r2, keep2 = ga.make_rope_params(headDim=64, offset=2**31 - 3)
    assert _rope_raw(r2, 4, 128, A, 2 * A) == 2 and "offset" in ga.attn_last_error()
    del keep, keep2


def test_rope_cache_write_refuses_before_launch():
    L = _lib.lib()
    A = 1 << 20
    r, keep = ga.make_rope_params(headDim=4)
    rr = ctypes.byref(r)
    assert L.attn_rope_cache_write(A, 10, 8, 2 * A, 3, 8, rr, None) == 1
    assert "offset" in ga.attn_last_error()
    assert L.attn_rope_cache_write(A, 10, 6, 2 * A, 1, 0, rr, None) == 1
    assert "headDim" in ga.attn_last_error()
    assert L.attn_rope_cache_write(None, 10, 8, 2 * A, 1, 0, rr, None) == 1
    assert "cache" in ga.attn_last_error()
    assert L.attn_rope_cache_write(A, 10, 8, A + 32, 2, 1, rr, None) == 1
    assert "overlap" in ga.attn_last_error()
    assert L.attn_rope_cache_write(A, 10, 8, 2 * A, 1, 0, None, None) == 1
    assert "rope" in ga.attn_last_error()
    assert L.attn_rope_cache_write(A, 10, 8, 2 * A, 0, 10, rr, None) == 0  # rows = 0: no-op
    del keep


def test_q_rope_is_validated_with_the_attention_params():
    ga.attn_validate(1, 64, heads=8, kvHeads=2, headDim=64, posOffset=63, q_rope=dict(base=1e4))
    with pytest.raises(ga.AttnError) as e:
        ga.attn_validate(1, 64, heads=8, headDim=64, q_rope=dict(headDim=32))
    assert "q_rope.headDim" in e.value.message
    with pytest.raises(ga.AttnError) as e:
        ga.attn_validate(1, 64, heads=8, headDim=64, q_rope=dict(rotaryDim=80))
    assert "rotaryDim" in e.value.message
    with pytest.raises(ga.AttnError) as e:
        ga.attn_validate(1, 64, heads=8, headDim=64, q_rope=dict(scaling=dict(rope_type="linear")))
    assert "factor" in e.value.message


def test_table_cache_never_serves_a_stale_table():
    # The library keeps the last resolved table per thread. Alternate every
    # case, change an explicit table's contents in place at the same address,
    # and move the sequence length across dynamic scaling's threshold.
    order = list(range(len(TABLE_CASES))) * 2
    np.random.default_rng(5).shuffle(order)
    for i in order:
        name, kw, rows = TABLE_CASES[i]
        test_library_table_is_the_oracles_bit_for_bit(name, kw, rows)
        test_library_table_is_the_oracles_bit_for_bit(name, kw, rows)   # a cache hit
    L = _lib.lib()
    r, keep = ga.make_rope_params(headDim=8, invFreq=[1.0, 0.5, 0.25, 0.125])
    inv = (ctypes.c_float * 4)()
    af = ctypes.c_float()
    assert L.attn_rope_table(ctypes.byref(r), 1, inv, ctypes.byref(af)) == 0
    assert list(inv) == [1.0, 0.5, 0.25, 0.125]
    keep[0][2] = 3.0                                    # same pointer, new contents
    assert L.attn_rope_table(ctypes.byref(r), 1, inv, ctypes.byref(af)) == 0
    assert list(inv) == [1.0, 0.5, 3.0, 0.125]
    dyn = dict(headDim=64, scaling=dict(rope_type="dynamic", factor=2.0,
                                        original_max_position_embeddings=4096))
    for rows in (10, 5000, 4096, 4097, 10):
        got, _ = ga.attn_rope_table(rows=rows, **dyn)
        want, _ = oracle.rope_table(64, scaling=dyn["scaling"], seq_len=rows)
        np.testing.assert_array_equal(got, want)
