"""The matrix-core decode kernel (decode_mfma) against the oracle, on the GPU.

decode_mfma serves decode-shaped calls whose KV groups hold many query rows
(several heads per KV head, or a few query rows of each): it reads every
visible K and V row once per group, like decode_split, and runs both
contractions on the matrix cores. Each case forces it with the
`decode_mfma` option (1) and checks every output element against the f64
oracle at |gpu - ref| <= 1e-4 + 1e-4 |ref|; where decode_split can serve the
same call, both kernels are run.
"""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import oracle
import workloads
from tests.parity import assert_close, compare, dev, run_library, torch

pytestmark = pytest.mark.gpu

BIAS_KIND = {None: 0, "TS": 1, "HTS": 2}


@pytest.fixture
def mfma():
    ga.attn_set_option("decode_mfma", 1)
    yield
    ga.attn_set_option("decode_mfma", 0)


def _wl(**kw):
    base = dict(name="decode_mfma case", T=1, S=1000, heads=8, kvHeads=1, headDim=128)
    base.update(kw)
    if "posOffset" not in kw and base.get("causal", True):
        base["posOffset"] = base["S"] - base["T"]
    return workloads.Workload(**base)


def _run(w, what=None):
    q, k, v, bias = w.tensors()
    plan = ga.attn_plan(w.T, w.S, bias_kind=BIAS_KIND[w.bias], **w.params())
    assert plan["path"] == "decode" and plan["variant"] == 1, plan
    return compare(q, k, v, bias, w.params(), what=what or w.name)


# Rows per KV group from 1 to 32 (two row blocks), ragged in both the rows
# and the key range.
@pytest.mark.parametrize("D, Dv", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("H, G, T", [(8, 8, 1), (12, 4, 1), (8, 2, 1), (7, 1, 1), (8, 1, 1), (12, 1, 1),
                                     (16, 1, 1), (8, 1, 2), (32, 2, 1), (24, 1, 1), (8, 1, 4), (64, 8, 1)])
def test_mfma_decode_shapes(D, Dv, H, G, T, mfma):
    rows = T * H // G
    if rows > {64: 32, 128: 32, 192: 16}[D]:
        pytest.skip("more rows per group than this width's instance holds")
    w = _wl(T=T, S=777, heads=H, kvHeads=G, headDim=D, vHeadDim=Dv, seed=D + H + T)
    _run(w)


@pytest.mark.parametrize("feature", [
    dict(window=100), dict(window=1), dict(softcap=5.0, std=3.0), dict(alibi=True),
    dict(alibiMax=16.0), dict(alibiSlopes=tuple(0.01 * (h + 1) for h in range(8))),
    dict(bias="TS", bias_mask_prob=0.1), dict(bias="HTS", bias_mask_prob=0.3),
    dict(scale=0.03), dict(causal=False), dict(causal=False, window=50, posOffset=500),
    dict(window=300, sinks=5), dict(causal=False, window=40, posOffset=300, sinks=3),
    dict(softcap=20.0, window=300, alibi=True, bias="HTS", bias_mask_prob=0.1, std=2.0),
])
@pytest.mark.parametrize("T", [1, 3])
def test_mfma_decode_features(feature, T, mfma):
    w = _wl(T=T, **feature)
    q, k, v, bias = w.tensors()
    if bias is not None:
        bias[..., 0] = 0.0  # key 0 stays unmasked
    plan = ga.attn_plan(w.T, w.S, bias_kind=BIAS_KIND[w.bias], **w.params())
    assert plan["variant"] == 1, plan
    compare(q, k, v, bias, w.params(), what=f"{feature} T={T}")


def test_mfma_two_row_blocks_with_epilogue(mfma):
    # 24 rows per group (two blocks of 16) with softcap, ALiBi and a bias.
    w = _wl(T=3, heads=16, kvHeads=2, S=2000, softcap=25.0, alibi=True, bias="HTS", bias_mask_prob=0.1,
            std=2.0)
    _run(w)


@pytest.mark.parametrize("splits", [1, 2, 5, 16, 64])
def test_mfma_split_count_does_not_change_the_result(splits, mfma):
    w = _wl(S=4000, heads=64, kvHeads=8)
    q, k, v, _ = w.tensors()
    try:
        ga.attn_set_option("decode_splits", splits)
        got1 = compare(q, k, v, None, w.params(), what=f"splits={splits}")
        got2 = run_library(q, k, v, None, w.params()).cpu().numpy()
    finally:
        ga.attn_set_option("decode_splits", 0)
    np.testing.assert_array_equal(got1.view(np.uint32), got2.view(np.uint32))


WALK_CASES = [
    dict(S=4000, heads=64, kvHeads=8),
    dict(S=1001, heads=16, kvHeads=2),                                      # ragged last block
    dict(S=3000, heads=16, kvHeads=2, window=1234),                         # window start mid-block
    dict(S=3000, posOffset=1500, heads=16, kvHeads=2, causal=False, window=700),
    dict(S=5000, heads=16, kvHeads=2, window=2100, sinks=5),                # sink split after the blocks
    dict(S=2000, heads=16, kvHeads=2, headDim=192, vHeadDim=128, alibi=True, bias="HTS", bias_mask_prob=0.2),
    dict(S=2500, T=3, heads=16, kvHeads=8),                                 # rows see different keys
    dict(S=100, heads=16, kvHeads=1, headDim=64),                           # fewer blocks than splits
]


@pytest.mark.parametrize("block", [-1, 32, 64, 512, 1024])
@pytest.mark.parametrize("case", range(len(WALK_CASES)))
def test_mfma_walks_agree(block, case, mfma):
    w = _wl(**WALK_CASES[case], seed=case)
    q, k, v, bias = w.tensors()
    try:
        ga.attn_set_option("decode_block", block)
        got1 = compare(q, k, v, bias, w.params(), what=f"block={block} {WALK_CASES[case]}")
        got2 = run_library(q, k, v, bias, w.params()).cpu().numpy()
    finally:
        ga.attn_set_option("decode_block", 0)
    np.testing.assert_array_equal(got1.view(np.uint32), got2.view(np.uint32))


def test_mfma_never_reads_rows_past_the_position(mfma):
    w = _wl(S=2048, posOffset=1499, heads=64, kvHeads=8)
    q, k, v, _ = w.tensors()
    k[1500:] = np.nan
    v[1500:] = np.nan
    got = compare(q, k, v, None, w.params(), what="poisoned tail")
    assert np.isfinite(got).all()
    k[:900] = np.nan
    v[:900] = np.nan
    compare(q, k, v, None, dict(w.params(), window=600), what="poisoned head outside window")


def test_mfma_empty_rows_are_zero(mfma):
    # Rows at positions 3, 4, 5 with window 2 over 4 keys: the last row of
    # each head sees nothing and comes out 0.
    w = _wl(T=3, S=4, posOffset=3, heads=8, kvHeads=2, headDim=64, window=2)
    got = _run(w, what="empty row")
    assert np.all(got[2] == 0.0)


def test_mfma_matches_decode_split_where_both_serve():
    # 8 rows per group at D=128 (both kernels hold them): each against the
    # oracle, and the two within the bar of each other.
    w = _wl(S=6000, heads=32, kvHeads=4, alibi=True, softcap=30.0)
    q, k, v, _ = w.tensors()
    got = {}
    try:
        for opt in (1, -1):
            ga.attn_set_option("decode_mfma", opt)
            plan = ga.attn_plan(w.T, w.S, **w.params())
            assert plan["variant"] == (1 if opt == 1 else 0), plan
            got[opt] = compare(q, k, v, None, w.params(), what=f"decode_mfma={opt}")
    finally:
        ga.attn_set_option("decode_mfma", 0)
    assert_close(got[1], got[-1].astype(np.float64), "decode_mfma vs decode_split")


def test_mfma_with_rotary_q(mfma):
    w = _wl(S=640, heads=32, kvHeads=4)
    qr = dict(base=500000.0, scaling=dict(rope_type="llama3", factor=8.0, low_freq_factor=1.0,
                                          high_freq_factor=4.0, original_max_position_embeddings=8192))
    q, k, v, _ = w.tensors()
    roped = oracle.rope(q, headDim=w.headDim, offset=w.posOffset, **qr).astype(np.float32)
    ref = oracle.attention(roped, k, v, **w.params())
    out = ga.attn_forward(dev(q), dev(k), dev(v), q_rope=dict(qr), **w.params())
    torch().cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "decode_mfma with q_rope")


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("kw, rows", [
    (dict(S=4096, heads=64, kvHeads=8), 1),
    (dict(S=1000, T=2, heads=16, kvHeads=2, alibi=True, bias="TS"), 2),
    (dict(S=700, heads=16, kvHeads=1, headDim=192, vHeadDim=128, window=100, sinks=2), 1),
    (dict(S=1200, heads=8, kvHeads=1), 17),
])
def test_mfma_fused_append(kw, rows, mfma):
    # attn_forward_append on decode_mfma: the new rows are read from their
    # buffers, stored into the caches by the kernel (bit for bit) and
    # attended. The rows being written hold NaN in the caches beforehand.
    t = torch()
    w = _wl(**kw)
    q, k, v, bias = w.tensors()
    offset = w.S - rows
    kc, vc = dev(k), dev(v)
    kc[offset:] = float("nan")
    vc[offset:] = float("nan")
    plan = ga.attn_plan(w.T, w.S, bias_kind=BIAS_KIND[w.bias], **w.params())
    assert plan["variant"] == 1, plan
    ga.attn_timing_enable(True)
    try:
        ga.attn_timing_collect("cache_write")
        out = ga.attn_forward_append(dev(q), kc, vc, dev(k[offset:]), dev(v[offset:]), offset, dev(bias),
                                     **w.params())
        t.cuda.synchronize()
        _, copies = ga.attn_timing_collect("cache_write")
    finally:
        ga.attn_timing_enable(False)
    assert copies == 0, "the append should run inside decode_mfma"
    np.testing.assert_array_equal(_bits(kc), k.view(np.uint32))
    np.testing.assert_array_equal(_bits(vc), v.view(np.uint32))
    assert_close(out.cpu().numpy(), oracle.attention(q, k, v, bias, **w.params()), str(kw))


@pytest.mark.parametrize("w", [workloads.LLAMA70_DECODE, workloads.QWEN2_DECODE], ids=["64-8", "28-4"])
def test_wide_group_decode_full_size_automatic(w):
    # The automatic choice for 8 (or 7) rows per group at D=128 is decode_mfma.
    plan = ga.attn_plan(w.T, w.S, **w.params())
    assert plan["path"] == "decode" and plan["variant"] == 1, plan
    q, k, v, _ = w.tensors()
    compare(q, k, v, None, w.params(), what=w.name)
