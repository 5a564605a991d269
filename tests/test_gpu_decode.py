"""Decode path (split-S + combine) against the oracle, on the GPU."""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import workloads
from tests.parity import assert_close, compare, dev, run_library, torch
import oracle

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(name="decode case", T=1, S=1000, heads=8, kvHeads=2, headDim=128, posOffset=999)
    base.update(kw)
    return workloads.Workload(**base)


def _check(w, what=None, expect_path="decode"):
    q, k, v, bias = w.tensors()
    params = w.params()
    plan = ga.attn_plan(w.T, w.S, bias_kind={None: 0, "TS": 1, "HTS": 2}[w.bias], **params)
    assert plan["path"] == expect_path, plan
    compare(q, k, v, bias, params, what=what or w.name)


@pytest.mark.parametrize("D, Dv", [(64, 64), (128, 128), (192, 128), (256, 256)])
@pytest.mark.parametrize("H, G, T", [(8, 2, 1), (16, 16, 1), (8, 4, 1), (4, 1, 1), (8, 8, 2), (6, 3, 1), (8, 8, 3),
                                     (16, 2, 1), (64, 8, 1), (28, 4, 1), (7, 1, 1), (12, 4, 2)])
def test_decode_shapes(D, Dv, H, G, T):
    nq = T * H // G
    if nq > {64: 8, 128: 8, 192: 4, 256: 2}[D]:
        pytest.skip("more query rows per group than this width's decode instance holds")
    S = 777
    w = _wl(T=T, S=S, heads=H, kvHeads=G, headDim=D, vHeadDim=Dv, posOffset=S - T, seed=D + H + T)
    _check(w)


@pytest.mark.parametrize("feature", [
    dict(window=100), dict(window=1), dict(softcap=5.0, std=3.0), dict(alibi=True),
    dict(alibiMax=16.0), dict(alibiSlopes=tuple(0.01 * (h + 1) for h in range(8))),
    dict(bias="TS", bias_mask_prob=0.1), dict(bias="HTS", bias_mask_prob=0.3),
    dict(scale=0.03), dict(causal=False), dict(causal=False, window=50, posOffset=500),
    dict(softcap=20.0, window=300, alibi=True, bias="HTS", bias_mask_prob=0.1, std=2.0),
])
def test_decode_features(feature):
    w = _wl(**feature)
    _check(w, what=str(feature))


@pytest.mark.parametrize("splits", [1, 2, 5, 16, 64])
def test_decode_split_count_does_not_change_the_result(splits):
    w = _wl(S=4000, posOffset=3999, heads=32, kvHeads=8)
    q, k, v, _ = w.tensors()
    try:
        ga.attn_set_option("decode_splits", splits)
        assert ga.attn_plan(1, 4000, **w.params())["splits"] == min(splits, (4000 + 63) // 64)
        got1 = compare(q, k, v, None, w.params(), what=f"splits={splits}")
        got2 = run_library(q, k, v, None, w.params()).cpu().numpy()
    finally:
        ga.attn_set_option("decode_splits", 0)
    np.testing.assert_array_equal(got1.view(np.uint32), got2.view(np.uint32))


def test_decode_never_reads_rows_past_the_position():
    # A cache of 2048 rows of which only 1500 are written; the rest is NaN.
    t = torch()
    w = _wl(S=2048, posOffset=1499, heads=32, kvHeads=8, T=1)
    q, k, v, _ = w.tensors()
    k[1500:] = np.nan
    v[1500:] = np.nan
    got = compare(q, k, v, None, w.params(), what="poisoned tail")
    assert np.isfinite(got).all()
    # Also when the window start is in the middle of the written part.
    k[:900] = np.nan
    v[:900] = np.nan
    compare(q, k, v, None, dict(w.params(), window=600), what="poisoned head outside window")
    del t


def test_decode_multi_row_with_an_empty_row():
    # Rows at positions 3, 4, 5 with window 2 over 4 keys: the last row sees nothing.
    w = _wl(T=3, S=4, posOffset=3, heads=2, kvHeads=1, headDim=64, window=2)
    q, k, v, _ = w.tensors()
    got = compare(q, k, v, None, w.params(), what="empty row")
    assert np.all(got[2] == 0.0)


def test_decode_output_guard_bands_untouched():
    t = torch()
    w = _wl(heads=32, kvHeads=8)
    q, k, v, _ = w.tensors()
    n, pad = w.T * 32 * 128, 64
    big = t.full((n + 2 * pad,), float("nan"), dtype=t.float32, device="cuda")
    out = big[pad:pad + n].view(w.T, 32 * 128)
    compare(q, k, v, None, w.params(), out=out, what="guarded out")
    b = big.cpu().numpy()
    assert np.isnan(b[:pad]).all() and np.isnan(b[-pad:]).all()


def test_llama_decode_full_size():
    # T=1 against a 32768-row cache filled through cache_write, posOffset 32767.
    t = torch()
    w = workloads.LLAMA_DECODE
    q, k, v, _ = w.tensors()
    kc = t.full(k.shape, float("nan"), dtype=t.float32, device="cuda")
    vc = t.full(v.shape, float("nan"), dtype=t.float32, device="cuda")
    kd, vd = dev(k), dev(v)
    ga.attn_cache_write(kc, kd[:-1], 0)
    ga.attn_cache_write(vc, vd[:-1], 0)
    ga.attn_cache_write(kc, kd[-1:], w.S - 1)
    ga.attn_cache_write(vc, vd[-1:], w.S - 1)
    got = ga.attn_forward(dev(q), kc, vc, **w.params())
    t.cuda.synchronize()
    ref = oracle.attention(q, k, v, **w.params())
    assert_close(got.cpu().numpy(), ref, w.name)


@pytest.mark.parametrize("w", [workloads.LLAMA70_DECODE, workloads.QWEN2_DECODE], ids=["64-8", "28-4"])
def test_wide_group_decode_full_size(w):
    # 8 (or 7) query heads per KV head take the decode path, all rows of a
    # group in one workgroup; every output element against the oracle.
    plan = ga.attn_plan(w.T, w.S, **w.params())
    assert plan["path"] == "decode", plan
    _check(w)


def test_latent_alibi_bias_decode_full_size():
    w = workloads.LATENT_DECODE
    _check(w)


def test_decode_is_deterministic():
    w = _wl(S=5000, posOffset=4999, heads=32, kvHeads=8, alibi=True, softcap=30.0)
    q, k, v, _ = w.tensors()
    a = run_library(q, k, v, None, w.params()).cpu().numpy()
    b = run_library(q, k, v, None, w.params()).cpu().numpy()
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_one_workspace_serves_every_shape_and_path():
    # One workspace (left holding garbage between calls) reused by decode calls
    # of several shapes and split counts and by a key-split prefill, in any
    # order: every call must give the oracle's result.
    t = torch()
    ws = t.full((64 << 20,), 0x7F, dtype=t.uint8, device="cuda")
    cases = [
        _wl(S=5000, posOffset=4999, heads=32, kvHeads=8),
        _wl(S=3000, posOffset=2999, heads=16, kvHeads=16, headDim=192, vHeadDim=128, bias="HTS",
            bias_mask_prob=0.1),
        workloads.Workload("split prefill", T=70, S=900, heads=8, kvHeads=2, headDim=128, posOffset=830),
        _wl(S=9000, posOffset=8999, heads=8, kvHeads=1, headDim=64),
    ]
    for rep in range(2):
        for w in cases:
            q, k, v, bias = w.tensors()
            got = ga.attn_forward(dev(q), dev(k), dev(v), dev(bias), workspace=ws, **w.params())
            t.cuda.synchronize()
            assert_close(got.cpu().numpy(), oracle.attention(q, k, v, bias, **w.params()), w.name)


WALK_CASES = [
    dict(S=4000, posOffset=3999, heads=32, kvHeads=8),
    dict(S=1001, posOffset=1000, heads=8, kvHeads=2),                       # ragged last block
    dict(S=3000, posOffset=2999, heads=8, kvHeads=2, window=1234),          # window start mid-block
    dict(S=3000, posOffset=1500, heads=8, kvHeads=2, causal=False, window=700),
    dict(S=5000, posOffset=4999, heads=8, kvHeads=2, window=2100, sinks=5),  # sink split after the blocks
    dict(S=2000, posOffset=1999, heads=16, kvHeads=16, headDim=192, vHeadDim=128, alibi=True,
         bias="HTS", bias_mask_prob=0.2),
    dict(S=2500, posOffset=2497, T=3, heads=8, kvHeads=8),                  # rows see different keys: chunks
    dict(S=100, posOffset=99, heads=4, kvHeads=1, headDim=64),              # fewer blocks than splits
]


@pytest.mark.parametrize("block", [-1, 32, 64, 1024])
@pytest.mark.parametrize("case", range(len(WALK_CASES)))
def test_decode_split_walks_agree(block, case):
    # Chunks per split (block -1) or interleaved blocks of `block` rows: both
    # cover every visible key once; each against the oracle, and each
    # deterministic.
    w = _wl(**WALK_CASES[case], seed=case)
    q, k, v, bias = w.tensors()
    try:
        ga.attn_set_option("decode_block", block)
        got1 = compare(q, k, v, bias, w.params(), what=f"block={block} {WALK_CASES[case]}")
        got2 = run_library(q, k, v, bias, w.params()).cpu().numpy()
    finally:
        ga.attn_set_option("decode_block", 0)
    np.testing.assert_array_equal(got1.view(np.uint32), got2.view(np.uint32))


@pytest.mark.parametrize("splits", [3, 7, 64])
def test_decode_interleaved_blocks_with_forced_splits(splits):
    # 4000 keys in blocks of 32 (125 blocks): split counts that do not
    # divide them leave splits with one block more than others.
    w = _wl(S=4000, posOffset=3999, heads=32, kvHeads=8, seed=splits)
    q, k, v, _ = w.tensors()
    try:
        ga.attn_set_option("decode_splits", splits)
        compare(q, k, v, None, w.params(), what=f"interleaved, splits={splits}")
    finally:
        ga.attn_set_option("decode_splits", 0)


DEPTH_CASES = [
    dict(S=3001, posOffset=3000, heads=32, kvHeads=8),
    dict(S=2000, posOffset=1999, heads=16, kvHeads=16, headDim=192, vHeadDim=128, alibi=True, bias="HTS",
         bias_mask_prob=0.2),
    dict(S=1500, posOffset=1499, heads=16, kvHeads=2, headDim=64),
    dict(S=1500, posOffset=1499, heads=4, kvHeads=2, headDim=256, window=700, sinks=3),
    dict(S=900, posOffset=898, T=2, heads=8, kvHeads=4, softcap=20.0),
]


@pytest.mark.parametrize("depth", [1, 2, 3])
@pytest.mark.parametrize("case", range(len(DEPTH_CASES)))
def test_decode_ring_depths(depth, case):
    # One batch per lane at a time (depth 1, the default) or a ring of 2 or 3
    # (where it fits; else 2): every depth against the oracle.
    w = _wl(**DEPTH_CASES[case], seed=40 + case)
    q, k, v, bias = w.tensors()
    got = {}
    try:
        for d in (1, depth):
            ga.attn_set_option("decode_depth", d)
            got[d] = compare(q, k, v, bias, w.params(), what=f"depth={d} {DEPTH_CASES[case]}")
    finally:
        ga.attn_set_option("decode_depth", 0)
