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
