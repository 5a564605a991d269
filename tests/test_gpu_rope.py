"""Rotary embedding on the GPU (op `rope`): standalone, rotate-then-write into
a KV cache, and fused into attention's q loads, against the oracle.

Bar for rope outputs (f32 result against the f64 oracle): every element
within ROPE_ATOL + ROPE_RTOL * |ref|. The kernel's cos and sin carry about
1.5e-7 absolute error (the angle is reduced in double precision, then rounded
to f32; the Taylor terms add f32 rounding), so an element a*cos - b*sin of
unit-scale inputs is off by a few 1e-7; 4e-6 leaves a wide margin while a
wrong pair, sign, frequency or position gives errors of order 1. Attention
outputs keep the attention bar (1e-4 + 1e-4 |ref|).
"""

import zlib

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import oracle
import workloads
from gqa_scaled_dot_amd import _lib
from tests.parity import assert_close, dev, torch

pytestmark = pytest.mark.gpu

ROPE_ATOL = 4e-6
ROPE_RTOL = 4e-6


def rope_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    bound = ROPE_ATOL + ROPE_RTOL * np.abs(ref)
    if (err > bound).any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: |err| {err[i]:.3e} > {bound[i]:.3e} at {i}")
    return float(err.max()) if err.size else 0.0


def oracle_kw(kw):
    return {k: kw[k] for k in ("headDim", "base", "offset", "rotaryDim", "interleaved", "scaling",
                               "invFreq", "attentionFactor") if k in kw}


LLAMA3 = dict(rope_type="llama3", factor=8.0, low_freq_factor=1.0, high_freq_factor=4.0,
              original_max_position_embeddings=8192)
YARN = dict(rope_type="yarn", factor=4.0, original_max_position_embeddings=4096)

# (T, heads, rope params); the vector kernel takes head widths that are
# multiples of 4 with rotaryDim % 8 == 0 (half-split) or % 4 == 0
# (interleaved); the rest go to the scalar kernel.
ROPE_CASES = [
    ("llama-decode-row", 1, 32, dict(headDim=128, base=500000.0, offset=32767)),
    ("llama3-scaled", 37, 8, dict(headDim=128, base=500000.0, offset=100, scaling=LLAMA3)),
    ("interleaved", 9, 4, dict(headDim=64, offset=5, interleaved=True)),
    ("partial-half", 16, 6, dict(headDim=96, rotaryDim=32, offset=1000)),
    ("partial-interleaved", 16, 6, dict(headDim=64, rotaryDim=20, interleaved=True, offset=3)),
    ("yarn-factor", 20, 2, dict(headDim=64, offset=70000, scaling=YARN)),
    ("huge-positions", 3, 4, dict(headDim=128, offset=2**31 - 10)),
    ("scalar-odd-width", 11, 3, dict(headDim=10, rotaryDim=6, offset=17)),
    ("scalar-rd-not-8", 7, 5, dict(headDim=128, rotaryDim=4, offset=40)),
    ("scalar-interleaved", 5, 2, dict(headDim=6, interleaved=True, offset=9)),
    ("explicit-table", 4, 2, dict(headDim=16, invFreq=[1.5 ** -i for i in range(8)],
                                  attentionFactor=0.8, offset=12)),
    ("many-rows", 4096, 8, dict(headDim=128, base=10000.0)),
]


@pytest.mark.parametrize("name, T, H, kw", ROPE_CASES, ids=[c[0] for c in ROPE_CASES])
def test_rope_matches_oracle(name, T, H, kw):
    x = workloads.normal((T, H * kw["headDim"]), 11, 0)
    got = ga.attn_rope(dev(x), **kw)
    torch().cuda.synchronize()
    ref = oracle.rope(x, **oracle_kw(kw))
    rope_close(got.cpu().numpy(), ref, name)
    rd = kw.get("rotaryDim") or kw["headDim"]
    # pass-through channels are copied bit for bit
    g = got.cpu().numpy().reshape(T, H, kw["headDim"])[..., rd:]
    np.testing.assert_array_equal(g.view(np.uint32),
                                  x.reshape(T, H, kw["headDim"])[..., rd:].view(np.uint32))


@pytest.mark.parametrize("kw", [dict(headDim=128, offset=77), dict(headDim=10, rotaryDim=6, offset=3),
                                dict(headDim=64, interleaved=True, rotaryDim=48)])
def test_rope_in_place_equals_out_of_place(kw):
    x = workloads.normal((50, 4 * kw["headDim"]), 12, 0)
    a = ga.attn_rope(dev(x), **kw)
    xd = dev(x)
    b = ga.attn_rope(xd, out=xd, **kw)
    torch().cuda.synchronize()
    assert b is xd
    np.testing.assert_array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


def test_rope_of_no_rows_is_a_no_op():
    t = torch()
    x = t.empty((0, 128), dtype=t.float32, device="cuda")
    out = ga.attn_rope(x, headDim=64)
    assert out.shape == (0, 128)


@pytest.mark.parametrize("rows, offset, rope_offset", [(1, 0, None), (1, 4095, None), (7, 100, None),
                                                       (16, 30, 1000)])
@pytest.mark.parametrize("width, D", [(1024, 128), (3072, 192), (30, 10)])
def test_rope_cache_write(rows, offset, rope_offset, width, D):
    max_rows = 4096 if offset >= 4000 else 200
    cache_np = workloads.normal((max_rows, width), 13, 1)
    cache = dev(cache_np)
    vals = workloads.normal((rows, width), 13, 2)
    kw = dict(headDim=D, base=500000.0)
    if rope_offset is not None:
        kw["offset"] = rope_offset
    out = ga.attn_rope_cache_write(cache, dev(vals), offset, kw)
    torch().cuda.synchronize()
    assert out is cache
    after = cache.cpu().numpy()
    ref = oracle.rope(vals, headDim=D, base=500000.0,
                      offset=offset if rope_offset is None else rope_offset)
    rope_close(after[offset:offset + rows], ref, "written rows")
    np.testing.assert_array_equal(after[:offset].view(np.uint32), cache_np[:offset].view(np.uint32))
    np.testing.assert_array_equal(after[offset + rows:].view(np.uint32),
                                  cache_np[offset + rows:].view(np.uint32))


# ---- rope fused into attention's q loads -------------------------------------

PATHS = {"decode": _lib.ATTN_PATH_DECODE, "prefill": _lib.ATTN_PATH_PREFILL,
         "generic": _lib.ATTN_PATH_GENERIC}

FUSED_CASES = [
    # (name, T, S, attention params, q_rope params, paths)
    ("llama-decode", 1, 3000, dict(heads=32, kvHeads=8, headDim=128, posOffset=2999),
     dict(base=500000.0, scaling=LLAMA3), ("decode", "prefill", "generic")),
    ("gqa-decode-interleaved", 2, 700, dict(heads=8, kvHeads=2, headDim=64, posOffset=698),
     dict(interleaved=True), ("decode", "prefill", "generic")),
    ("latent-decode-partial", 1, 900, dict(heads=16, headDim=192, vHeadDim=128, posOffset=899,
                                           alibi=True), dict(rotaryDim=64), ("decode", "generic")),
    ("prefill-128", 150, 150, dict(heads=8, kvHeads=2, headDim=128, softcap=20.0),
     dict(base=10000.0), ("prefill", "generic")),
    ("prefill-256-window", 130, 300, dict(heads=8, kvHeads=4, headDim=256, posOffset=170, window=60),
     dict(scaling=YARN), ("prefill", "generic")),
    ("prefill-192-partial-interleaved", 70, 70, dict(heads=4, headDim=192, vHeadDim=128),
     dict(rotaryDim=64, interleaved=True), ("prefill", "generic")),
]


def _attend(q, k, v, params, path, **extra):
    ga.attn_set_option("force_path", PATHS[path])
    try:
        out = ga.attn_forward(q, k, v, **params, **extra)
        torch().cuda.synchronize()
    finally:
        ga.attn_set_option("force_path", 0)
    return out.cpu().numpy()


@pytest.mark.parametrize("name, T, S, params, qr, paths", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_q_rope_matches_oracle_and_the_unfused_pair(name, T, S, params, qr, paths):
    w = workloads.Workload(name, T=T, S=S, seed=zlib.crc32(name.encode()) % 1000, **params)
    q, k, v, _ = w.tensors()
    D = w.headDim
    p0 = params.get("posOffset", 0)
    roped = oracle.rope(q, headDim=D, offset=p0, **qr).astype(np.float32)
    ref = oracle.attention(roped, k, v, **params)
    qd, kd, vd = dev(q), dev(k), dev(v)
    q_turned = ga.attn_rope(qd, headDim=D, offset=p0, **qr)
    for path in paths:
        fused = _attend(qd, kd, vd, params, path, q_rope=dict(qr))
        assert_close(fused, ref, f"{name} {path}")
        # The kernels turn q exactly as the rope kernel does: same bits out.
        unfused = _attend(q_turned, kd, vd, params, path)
        np.testing.assert_array_equal(fused.view(np.uint32), unfused.view(np.uint32))


def test_fused_q_rope_in_both_prefill_variants():
    w = workloads.Workload("variants", T=100, S=100, heads=8, kvHeads=2, headDim=128)
    q, k, v, _ = w.tensors()
    qr = dict(base=500000.0, offset=0)
    ref = oracle.attention(oracle.rope(q, headDim=128, **qr).astype(np.float32), k, v, **w.params())
    try:
        for variant in (32, 16):
            ga.attn_set_option("prefill_variant", variant)
            got = ga.attn_forward(dev(q), dev(k), dev(v), q_rope=qr, **w.params())
            assert_close(got.cpu().numpy(), ref, f"variant {variant}")
    finally:
        ga.attn_set_option("prefill_variant", 0)


def test_q_rope_offset_defaults_to_pos_offset():
    w = workloads.Workload("default offset", T=1, S=500, heads=8, kvHeads=8, headDim=64, posOffset=499)
    q, k, v, _ = w.tensors()
    a = ga.attn_forward(dev(q), dev(k), dev(v), q_rope=dict(), **w.params()).cpu().numpy()
    b = ga.attn_forward(dev(q), dev(k), dev(v), q_rope=dict(offset=499), **w.params()).cpu().numpy()
    c = ga.attn_forward(dev(q), dev(k), dev(v), q_rope=dict(offset=0), **w.params()).cpu().numpy()
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)


def test_llama_decode_step_with_rope_full_size():
    """One decode step of the Llama-shaped workload as a graph runs it: K rows
    turned and written by attn_rope_cache_write (the past rows, then the new
    one at 32767), V by cache_write, q turned inside attention."""
    w = workloads.LLAMA_DECODE
    q, k, v, _ = w.tensors()
    rp = dict(headDim=w.headDim, base=500000.0, scaling=LLAMA3)
    t = torch()
    kc = t.empty((w.S, w.G * w.headDim), dtype=t.float32, device="cuda")
    vc = t.empty((w.S, w.G * w.Dv), dtype=t.float32, device="cuda")
    kd, vd = dev(k), dev(v)
    ga.attn_rope_cache_write(kc, kd[:w.S - 1], 0, rp)
    ga.attn_cache_write(vc, vd[:w.S - 1], 0)
    ga.attn_rope_cache_write(kc, kd[w.S - 1:], w.S - 1, rp)
    ga.attn_cache_write(vc, vd[w.S - 1:], w.S - 1)
    got = ga.attn_forward(dev(q), kc, vc, q_rope=dict(base=500000.0, scaling=LLAMA3), **w.params())
    t.cuda.synchronize()
    k_rot = oracle.rope(k, offset=0, **rp)
    rope_close(kc.cpu().numpy(), k_rot, "rotated K cache")
    q_rot = oracle.rope(q, offset=w.posOffset, **rp).astype(np.float32)
    ref = oracle.attention(q_rot, k_rot.astype(np.float32), v, **w.params())
    assert_close(got.cpu().numpy(), ref, "llama decode with rope")


def test_llama_prefill_with_rope_sampled_rows():
    w = workloads.LLAMA_PREFILL
    q, k, v, _ = w.tensors()
    rp = dict(headDim=w.headDim, base=500000.0)
    t = torch()
    kc = t.empty((w.S, w.G * w.headDim), dtype=t.float32, device="cuda")
    ga.attn_rope_cache_write(kc, dev(k), 0, rp)
    got = ga.attn_forward(dev(q), kc, dev(v), q_rope=dict(base=500000.0), **w.params())
    t.cuda.synchronize()
    rows = [0, 1, 31, 32, 1000, 2047, 2048, 3333, 4094, 4095]
    k_rot = oracle.rope(k, offset=0, **rp).astype(np.float32)
    q_rot = np.stack([oracle.rope(q[r:r + 1], offset=r, **rp)[0] for r in rows]).astype(np.float32)
    q_full = np.zeros_like(q)
    q_full[rows] = q_rot
    ref = oracle.attention(q_full, k_rot, v, rows=rows, **w.params())
    assert_close(got.cpu().numpy()[rows], ref, "llama prefill with rope")
