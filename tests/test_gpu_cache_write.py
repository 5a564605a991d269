"""cache_write on the GPU: an exact copy into rows [offset, offset+rows), nothing else touched."""

import numpy as np
import pytest

import workloads
from tests.parity import dev, torch

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("width", [1024, 3072, 1023, 12, 3, 1])
@pytest.mark.parametrize("rows, offset", [(1, 0), (1, 37), (5, 60), (64, 0), (17, 83)])
def test_cache_write_is_bit_exact_and_confined(width, rows, offset):
    import gqa_scaled_dot_amd as ga
    max_rows = 100
    cache = dev(workloads.normal((max_rows, width), 7, 1))
    before = _bits(cache)
    vals_np = workloads.normal((rows, width), 7, 2)
    vals_np[0, 0] = np.float32(np.nan)      # bit patterns travel as they are
    vals_np[-1, -1] = np.float32(-0.0)
    vals = dev(vals_np)
    out = ga.attn_cache_write(cache, vals, offset)
    torch().cuda.synchronize()
    assert out is cache
    after = _bits(cache)
    np.testing.assert_array_equal(after[offset:offset + rows], vals_np.view(np.uint32))
    np.testing.assert_array_equal(after[:offset], before[:offset])
    np.testing.assert_array_equal(after[offset + rows:], before[offset + rows:])


@pytest.mark.parametrize("src_shift", [0, 1, 2, 3])
def test_cache_write_misaligned_source(src_shift):
    # A source that starts 4*src_shift bytes off the 16-byte phase of the destination.
    import gqa_scaled_dot_amd as ga
    width, rows, offset = 257, 9, 11
    cache = dev(np.zeros((40, width), np.float32))
    pool_np = workloads.normal((rows * width + 8,), 3, 2)
    pool = dev(pool_np)
    vals = pool[src_shift:src_shift + rows * width].view(rows, width)
    ga.attn_cache_write(cache, vals, offset)
    torch().cuda.synchronize()
    got = _bits(cache)
    want = pool_np[src_shift:src_shift + rows * width].reshape(rows, width).view(np.uint32)
    np.testing.assert_array_equal(got[offset:offset + rows], want)
    assert not got[:offset].any() and not got[offset + rows:].any()


def test_cache_write_fills_a_full_decode_cache():
    # The Llama-shaped cache: 32768 rows of 8 KV heads x 128, filled in one call,
    # then the last row appended on its own.
    import gqa_scaled_dot_amd as ga
    t = torch()
    S, width = 32768, 1024
    cache = t.full((S, width), float("nan"), dtype=t.float32, device="cuda")
    vals = dev(workloads.normal((S, width), 0, 1))
    ga.attn_cache_write(cache, vals[:S - 1], 0)
    ga.attn_cache_write(cache, vals[S - 1:], S - 1)
    t.cuda.synchronize()
    assert t.equal(cache.view(t.int32), vals.view(t.int32))


def test_cache_write_zero_rows_is_a_noop():
    import gqa_scaled_dot_amd as ga
    cache = dev(np.ones((4, 8), np.float32))
    vals = dev(np.zeros((0, 8), np.float32))
    ga.attn_cache_write(cache, vals, 4)
    torch().cuda.synchronize()
    assert np.all(cache.cpu().numpy() == 1.0)


def test_cache_write_refuses_out_of_range():
    import gqa_scaled_dot_amd as ga
    cache = dev(np.ones((4, 8), np.float32))
    vals = dev(np.zeros((2, 8), np.float32))
    with pytest.raises(ga.AttnError):
        ga.attn_cache_write(cache, vals, 3)
    torch().cuda.synchronize()
    assert np.all(cache.cpu().numpy() == 1.0)


@pytest.mark.parametrize("wa, wb", [(1024, 1024), (3072, 2048), (1023, 5), (12, 4096), (1, 3)])
@pytest.mark.parametrize("rows, offset", [(1, 0), (1, 99), (7, 40), (64, 36)])
def test_cache_write2_equals_two_cache_writes(wa, wb, rows, offset):
    # K and V rows in one launch: each cache ends up bit for bit as one
    # attn_cache_write leaves it, every other row untouched.
    import gqa_scaled_dot_amd as ga
    max_rows = 100
    ca = dev(workloads.normal((max_rows, wa), 11, 1))
    cb = dev(workloads.normal((max_rows, wb), 11, 2))
    before_a, before_b = _bits(ca), _bits(cb)
    va_np = workloads.normal((rows, wa), 11, 3)
    vb_np = workloads.normal((rows, wb), 11, 4)
    va_np[0, 0] = np.float32(np.nan)
    vb_np[-1, -1] = np.float32(-0.0)
    ra, rb = ga.attn_cache_write2(ca, dev(va_np), cb, dev(vb_np), offset)
    torch().cuda.synchronize()
    assert ra is ca and rb is cb
    for after, before, v in ((_bits(ca), before_a, va_np), (_bits(cb), before_b, vb_np)):
        np.testing.assert_array_equal(after[offset:offset + rows], v.view(np.uint32))
        np.testing.assert_array_equal(after[:offset], before[:offset])
        np.testing.assert_array_equal(after[offset + rows:], before[offset + rows:])


@pytest.mark.parametrize("shift_a, shift_b", [(0, 1), (3, 0), (2, 2), (1, 3)])
def test_cache_write2_misaligned_sources(shift_a, shift_b):
    # Sources off the destinations' 16-byte phase take the 32-bit copy; each
    # copy picks its own.
    import gqa_scaled_dot_amd as ga
    rows, offset, wa, wb = 5, 13, 257, 130
    ca = dev(np.zeros((30, wa), np.float32))
    cb = dev(np.zeros((30, wb), np.float32))
    pa_np = workloads.normal((rows * wa + 8,), 5, 1)
    pb_np = workloads.normal((rows * wb + 8,), 5, 2)
    pa, pb = dev(pa_np), dev(pb_np)
    va = pa[shift_a:shift_a + rows * wa].view(rows, wa)
    vb = pb[shift_b:shift_b + rows * wb].view(rows, wb)
    ga.attn_cache_write2(ca, va, cb, vb, offset)
    torch().cuda.synchronize()
    for got, p_np, w, sh in ((_bits(ca), pa_np, wa, shift_a), (_bits(cb), pb_np, wb, shift_b)):
        want = p_np[sh:sh + rows * w].reshape(rows, w).view(np.uint32)
        np.testing.assert_array_equal(got[offset:offset + rows], want)
        assert not got[:offset].any() and not got[offset + rows:].any()


def test_cache_write2_decode_append_then_attend():
    # The decode step's append: the new K and V rows at 32767 of the
    # Llama-shaped caches, then attention over them, against the oracle.
    import gqa_scaled_dot_amd as ga
    import oracle
    from tests.parity import assert_close
    t = torch()
    w = workloads.LLAMA_DECODE
    q, k, v, _ = w.tensors()
    kc = t.full(k.shape, float("nan"), dtype=t.float32, device="cuda")
    vc = t.full(v.shape, float("nan"), dtype=t.float32, device="cuda")
    kd, vd = dev(k), dev(v)
    ga.attn_cache_write2(kc, kd[:-1], vc, vd[:-1], 0)
    ga.attn_cache_write2(kc, kd[-1:], vc, vd[-1:], w.S - 1)
    got = ga.attn_forward(dev(q), kc, vc, **w.params())
    t.cuda.synchronize()
    assert_close(got.cpu().numpy(), oracle.attention(q, k, v, **w.params()), "cache_write2 then decode")
