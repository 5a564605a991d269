"""attn_forward_append on the GPU: a decode step's `cache_write` of its new K
and V rows and op `attention` over the caches, in one call.

The caches must come out as the copy leaves them, bit for bit (rows
[offset, offset + rows) are the new rows, every other row untouched), and
the output must meet the attention bar (|gpu - ref| <= 1e-4 + 1e-4 |ref|)
against the f64 oracle over the updated caches. Before the call the rows
being written hold NaN, so a kernel that read them from the caches instead
of the new-row buffers would fail; where the key range ends there, the rows
past it hold NaN too. The library's launch records tell whether the copy
ran in a launch of its own or inside the decode kernel.
"""

import numpy as np
import pytest

import gqa_scaled_dot_amd as ga
import oracle
import workloads
from tests.parity import assert_close, dev, torch

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


def _append(w, rows, offset, *, poison_past=None, shift=0, extra=None, ref_extra=None, what=""):
    """Run one appending call of workload w; check caches and output.
    Returns the number of separate copy launches (0: fused)."""
    t = torch()
    q, k, v, bias = w.tensors()
    kc, vc = dev(k), dev(v)
    kc[offset:offset + rows] = float("nan")
    vc[offset:offset + rows] = float("nan")
    if poison_past is not None:
        kc[poison_past:] = float("nan")
        vc[poison_past:] = float("nan")
    want_k, want_v = _bits(kc), _bits(vc)
    want_k[offset:offset + rows] = k[offset:offset + rows].view(np.uint32)
    want_v[offset:offset + rows] = v[offset:offset + rows].view(np.uint32)
    if shift:
        # New rows that start 4*shift bytes past a 16-byte boundary.
        pk = dev(np.concatenate([np.zeros(shift, np.float32), k[offset:offset + rows].ravel()]))
        pv = dev(np.concatenate([np.zeros(shift, np.float32), v[offset:offset + rows].ravel()]))
        kn = pk[shift:].view(rows, k.shape[1])
        vn = pv[shift:].view(rows, v.shape[1])
    else:
        kn, vn = dev(k[offset:offset + rows]), dev(v[offset:offset + rows])
    params = dict(w.params(), **(extra or {}))
    t.cuda.synchronize()
    ga.attn_timing_enable(True)
    try:
        ga.attn_timing_collect("cache_write")
        out = ga.attn_forward_append(dev(q), kc, vc, kn, vn, offset, dev(bias), **params)
        t.cuda.synchronize()
        _, copies = ga.attn_timing_collect("cache_write")
    finally:
        ga.attn_timing_enable(False)
    np.testing.assert_array_equal(_bits(kc), want_k)
    np.testing.assert_array_equal(_bits(vc), want_v)
    ref = oracle.attention(q, k, v, bias, **w.params(), **(ref_extra or {}))
    assert_close(out.cpu().numpy(), ref, what or w.name)
    return copies


def _wl(**kw):
    base = dict(name="append", T=1, S=300, heads=8, kvHeads=2, headDim=128)
    base.update(kw)
    if "posOffset" not in kw and base.get("causal", True):
        base["posOffset"] = base["S"] - base["T"]
    return workloads.Workload(**base)


# Decode steps whose new rows end the key range: one launch does both.
FUSED = [
    ("llama", dict(T=1, S=4096, heads=32, kvHeads=8)),
    ("T=4 causal masks on the new rows", dict(T=4, S=1000, heads=2, kvHeads=1, headDim=64)),
    ("T=2 G=2", dict(T=2, S=777, heads=4, kvHeads=2)),
    ("ALiBi softcap [T,S] bias", dict(S=2049, alibi=True, softcap=30.0, bias="TS", bias_mask_prob=0.1)),
    ("latent widths MPT [H,T,S] bias", dict(S=700, heads=16, kvHeads=4, headDim=192, vHeadDim=128,
                                            alibiMax=8.0, bias="HTS")),
    ("window and sinks", dict(S=5000, heads=32, kvHeads=8, window=256, sinks=4)),
    ("D=256", dict(S=3000, heads=8, kvHeads=4, headDim=256)),
    ("D=64 eight rows per group", dict(S=1500, heads=16, kvHeads=2, headDim=64, scale=0.3)),
    ("one key: the appended row", dict(S=1, posOffset=0)),
    ("first rows of a long cache", dict(S=4096, T=1, posOffset=0)),
]


@pytest.mark.parametrize("name, kw", FUSED, ids=[c[0] for c in FUSED])
def test_fused_decode_step(name, kw):
    w = _wl(name=name, **kw)
    bias_kind = {None: 0, "TS": 1, "HTS": 2}[w.bias]
    assert ga.attn_plan(w.T, w.S, bias_kind=bias_kind, **w.params())["path"] == "decode"
    rows = w.T
    offset = w.posOffset
    assert _append(w, rows, offset, poison_past=offset + rows) == 0


def test_fused_llama_decode_full_size():
    w = workloads.LLAMA_DECODE
    assert _append(w, 1, w.S - 1) == 0


def test_fused_non_causal_append_at_the_end():
    # Non-causal, no window: every row sees the whole cache; new rows at its end.
    w = _wl(S=900, causal=False, posOffset=0)
    assert _append(w, 3, w.S - 3) == 0


@pytest.mark.parametrize("rows", [2, 17, 64])
def test_fused_several_rows_for_one_query(rows):
    # A single query at the last of `rows` appended positions.
    w = _wl(S=1200)
    assert _append(w, rows, w.S - rows, what=f"rows={rows}") == 0


@pytest.mark.parametrize("opt, val", [("decode_splits", 1), ("decode_splits", 7), ("decode_block", 64),
                                      ("decode_depth", 2), ("decode_depth", 3), ("decode_wgs_per_cu", 1)])
def test_fused_under_plan_options(opt, val):
    w = _wl(S=8192, heads=32, kvHeads=8, alibi=True)
    try:
        ga.attn_set_option(opt, val)
        assert _append(w, 1, w.S - 1, what=f"{opt}={val}") == 0
    finally:
        ga.attn_set_option(opt, 0)


def test_fused_with_rotary_q():
    w = _wl(S=640)
    qr = dict(base=10000.0)
    q, k, v, bias = w.tensors()
    roped = oracle.rope(q, headDim=w.headDim, offset=w.posOffset, **qr).astype(np.float32)
    ref = oracle.attention(roped, k, v, **w.params())
    kc, vc = dev(k), dev(v)
    kc[-1] = float("nan")
    vc[-1] = float("nan")
    out = ga.attn_forward_append(dev(q), kc, vc, dev(k[-1:]), dev(v[-1:]), w.S - 1, q_rope=dict(qr), **w.params())
    torch().cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "rotary q")
    np.testing.assert_array_equal(_bits(kc), k.view(np.uint32))


FALLBACK = [
    # (name, workload, rows, offset, extra kwargs)
    ("rows before the end of the range", dict(S=500), 3, 480, {}),
    ("65 rows", dict(S=1200), 65, 1135, {}),
    ("rows below the window", dict(S=2000, window=100), 1, 1500, {}),
    ("prefill path", dict(T=200, S=400, heads=4, kvHeads=2, headDim=64), 200, 200, {}),
    ("generic path", dict(T=3, S=50, heads=4, kvHeads=2, headDim=16), 3, 47, {}),
    ("no key in view", dict(T=2, S=40, posOffset=100, causal=False, window=5), 4, 10, {}),
]


@pytest.mark.parametrize("name, kw, rows, offset, extra", FALLBACK, ids=[c[0] for c in FALLBACK])
def test_copy_first_where_the_rows_are_not_the_last_keys(name, kw, rows, offset, extra):
    w = _wl(name=name, **kw)
    assert _append(w, rows, offset, extra=extra) == 1


def test_copy_first_for_unaligned_new_rows():
    w = _wl(S=300)
    for shift in (1, 2, 3):
        assert _append(w, 1, w.S - 1, shift=shift, what=f"shift={shift}") == 1


def test_copy_first_with_position_bias():
    # Relative-position terms keep their own near split: the copy runs first.
    w = _wl(S=3000, heads=8, kvHeads=2)
    th = list(range(0, 320, 10))
    weight = workloads.normal((len(th), w.heads), 11, 0)
    assert _append(w, 1, w.S - 1, extra=dict(position_bias=dict(weight=dev(weight), buckets=th)),
                   ref_extra=dict(position_bias=dict(weight=weight, buckets=th))) == 1


def test_no_query_rows_only_writes():
    t = torch()
    k = workloads.normal((20, 256), 1, 1)
    v = workloads.normal((20, 256), 1, 2)
    kc = t.zeros((20, 256), device="cuda")
    vc = t.zeros((20, 256), device="cuda")
    q = t.zeros((0, 8 * 128), device="cuda")
    out = ga.attn_forward_append(q, kc, vc, dev(k[5:9]), dev(v[5:9]), 5, heads=8, kvHeads=2, headDim=128)
    t.cuda.synchronize()
    assert tuple(out.shape) == (0, 8 * 128)
    got = _bits(kc)
    np.testing.assert_array_equal(got[5:9], k[5:9].view(np.uint32))
    assert not got[:5].any() and not got[9:].any()
    np.testing.assert_array_equal(_bits(vc)[5:9], v[5:9].view(np.uint32))


def test_decode_loop_matches_separate_calls():
    # Twelve decode steps from position 500 on, through the fused call and
    # through cache_write2 + attn_forward on twin caches: same caches bit for
    # bit, outputs within the bar of each other and of the oracle.
    t = torch()
    w = _wl(S=512, heads=32, kvHeads=8, posOffset=499, alibi=True)
    q_all = workloads.normal((12, 32 * 128), 3, 0)
    k_all = workloads.normal((512, 8 * 128), 3, 1)
    v_all = workloads.normal((512, 8 * 128), 3, 2)
    ka, va = dev(k_all), dev(v_all)
    ka[500:] = float("nan")
    va[500:] = float("nan")
    kb, vb = ka.clone(), va.clone()
    params = dict(w.params())
    for i in range(12):
        pos = 500 + i
        params["posOffset"] = pos
        q = dev(q_all[i:i + 1])
        kn, vn = dev(k_all[pos:pos + 1]), dev(v_all[pos:pos + 1])
        fused = ga.attn_forward_append(q, ka, va, kn, vn, pos, **params)
        ga.attn_cache_write2(kb, kn, vb, vn, pos)
        sep = ga.attn_forward(q, kb, vb, **params)
        t.cuda.synchronize()
        assert t.equal(ka.view(t.int32), kb.view(t.int32)) and t.equal(va.view(t.int32), vb.view(t.int32))
        ref = oracle.attention(q_all[i:i + 1], k_all[:pos + 1], v_all[:pos + 1],
                               **dict(params, posOffset=pos))
        assert_close(fused.cpu().numpy(), ref, f"step {i}")
        assert_close(sep.cpu().numpy(), ref, f"step {i} separate")



@pytest.mark.parametrize("S, G, D", [(4097, 8, 128), (4721, 8, 128), (8193, 4, 128), (16385, 2, 128),
                                     (2321, 16, 64), (32769, 1, 64)])
def test_fused_within_the_reported_workspace(S, G, D):
    # Shapes where a range one row shorter rounds to more chunks: the call
    # still fits the workspace attn_workspace_size reports, and still fuses
    # (chunks are sized for the range with the appended row in it).
    t = torch()
    w = _wl(S=S, heads=2 * G, kvHeads=G, headDim=D)
    q, k, v, _ = w.tensors()
    ws = t.empty(ga.attn_workspace_size(w.T, w.S, **w.params()), dtype=t.uint8, device="cuda")
    kc, vc = dev(k), dev(v)
    kc[-1] = float("nan")
    vc[-1] = float("nan")
    ga.attn_timing_enable(True)
    try:
        ga.attn_timing_collect("cache_write")
        out = ga.attn_forward_append(dev(q), kc, vc, dev(k[-1:]), dev(v[-1:]), S - 1, workspace=ws, **w.params())
        t.cuda.synchronize()
        _, copies = ga.attn_timing_collect("cache_write")
    finally:
        ga.attn_timing_enable(False)
    assert copies == 0
    np.testing.assert_array_equal(_bits(kc), k.view(np.uint32))
    np.testing.assert_array_equal(_bits(vc), v.view(np.uint32))
    assert_close(out.cpu().numpy(), oracle.attention(q, k, v, **w.params()), f"S={S} G={G}")


def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    D, Dv, most = [(64, 64, 8), (128, 128, 4), (192, 128, 4), (256, 256, 2)][rng.integers(4)]
    G = int(rng.choice([1, 2, 4, 8]))
    T = int(rng.integers(1, 3))
    hpg = int(rng.choice([h for h in (1, 2, 4, 8) if h * T <= most] or [1]))
    T = 1 if hpg * T > most else T
    S = int(rng.integers(T, 6000))
    kw = dict(name=f"random append {seed}", T=T, S=S, heads=G * hpg, kvHeads=G, headDim=D, seed=seed)
    if Dv != D:
        kw["vHeadDim"] = Dv
    feats = rng.random(5)
    if feats[0] < 0.3:
        kw["alibi"] = True
    if feats[1] < 0.3:
        kw["softcap"] = 20.0
    if feats[2] < 0.3:
        kw["bias"] = "TS" if rng.random() < 0.5 else "HTS"
    if feats[3] < 0.3 and S > 100:
        kw["window"] = int(rng.integers(16, S))
        if feats[4] < 0.5:
            kw["sinks"] = int(rng.integers(1, 8))
    w = _wl(**kw)
    if rng.random() < 0.75:  # the step's own rows, at the end of the range
        rows = int(rng.integers(w.T, min(64, S) + 1)) if rng.random() < 0.3 else w.T
        rows = min(rows, w.posOffset + w.T)
        offset = w.posOffset + w.T - rows
    else:  # rows anywhere in the cache
        rows = int(rng.integers(1, min(80, S) + 1))
        offset = int(rng.integers(0, S - rows + 1))
    opts = {}
    if rng.random() < 0.25:
        opts[str(rng.choice(["decode_splits", "decode_block", "decode_depth"]))] = None
    for k in opts:
        opts[k] = {"decode_splits": int(rng.integers(1, 40)), "decode_block": 64, "decode_depth": 2}[k]
    return w, rows, offset, opts


@pytest.mark.parametrize("seed", range(40))
def test_random_appends(seed):
    w, rows, offset, opts = _random_case(seed)
    bias_kind = {None: 0, "TS": 1, "HTS": 2}[w.bias]
    assert ga.attn_plan(w.T, w.S, bias_kind=bias_kind, **w.params())["path"] == "decode", w
    try:
        for k, val in opts.items():
            ga.attn_set_option(k, val)
        _append(w, rows, offset, what=f"seed {seed}: rows {rows} at {offset} {opts} {w}")
    finally:
        for k in opts:
            ga.attn_set_option(k, 0)


def _random_noncausal_case(seed):
    """A non-causal appending call whose new rows end its key range: the
    cache's end without a window, else the last row's position + window + 1
    (rows past that hold NaN). Groups up to 16 rows (decode_mfma) where the
    width allows."""
    rng = np.random.default_rng(5000 + seed)
    D, Dv, most = [(64, 64, 16), (128, 128, 16), (192, 128, 16), (256, 256, 2)][rng.integers(4)]
    G = int(rng.choice([1, 2, 4, 8]))
    T = int(rng.integers(1, 3))
    hpg = int(rng.choice([h for h in (1, 2, 4, 7, 8) if h * T <= most] or [1]))
    S = int(rng.integers(T + 80, 6000))
    P0 = int(rng.integers(0, S - T + 1))
    kw = dict(name=f"random non-causal append {seed}", T=T, S=S, heads=G * hpg, kvHeads=G, headDim=D,
              causal=False, posOffset=P0, seed=seed)
    if Dv != D:
        kw["vHeadDim"] = Dv
    lo, end = 0, S
    if rng.random() < 0.6:
        window = int(rng.integers(1, S))
        kw["window"] = window
        lo, end = max(0, P0 - window), min(S, P0 + T + window)
        if rng.random() < 0.3:
            kw["sinks"] = int(rng.integers(1, 8))
    feats = rng.random(3)
    if feats[0] < 0.3:
        kw["alibi"] = True
    if feats[1] < 0.3:
        kw["softcap"] = 20.0
    if feats[2] < 0.3:
        kw["bias"] = "TS" if rng.random() < 0.5 else "HTS"
    w = _wl(**kw)
    rows = int(rng.integers(1, min(64, end - lo) + 1))
    return w, rows, end - rows, (end if end < S else None)


@pytest.mark.parametrize("seed", range(24))
def test_random_noncausal_appends(seed):
    # Non-causal calls whose appended rows end the key range take them into
    # the decode launch too (no separate copy); caches bit for bit, output
    # against the oracle.
    w, rows, offset, poison_past = _random_noncausal_case(seed)
    bias_kind = {None: 0, "TS": 1, "HTS": 2}[w.bias]
    assert ga.attn_plan(w.T, w.S, bias_kind=bias_kind, **w.params())["path"] == "decode", w
    copies = _append(w, rows, offset, poison_past=poison_past,
                     what=f"seed {seed}: rows {rows} at {offset}, rows from {poison_past} NaN; {w}")
    assert copies == 0
