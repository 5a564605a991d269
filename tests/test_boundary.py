"""The C-ABI boundary, checked on the CPU (no device calls).

The library must load, export every entry point include/attn.h declares,
resolve the op's defaults, and refuse bad arguments by name before any
launch (the catalogue rejects a graph that needs an unsupported feature and
names that feature).
"""

import ctypes
import os
import re
import subprocess

import pytest

import gqa_scaled_dot_amd as ga
from gqa_scaled_dot_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_binding_exports():
    assert set(_declared_functions()) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)", out))
    assert set(_declared_functions()) <= exported


def test_params_init_defaults():
    p = _lib.AttnParams()
    ctypes.memset(ctypes.byref(p), 0xFF, ctypes.sizeof(p))
    _lib.lib().attn_params_init(ctypes.byref(p))
    assert p.causal == 1
    assert (p.T, p.S, p.heads, p.kv_heads, p.head_dim, p.v_head_dim) == (0, 0, 0, 0, 0, 0)
    assert (p.pos_offset, p.window, p.has_scale, p.softcap, p.alibi, p.bias_kind) == (0, 0, 0, 0, 0, 0)
    assert not p.alibi_slopes and not p.q_rope and p.sinks == 0


BASE = dict(heads=8, kvHeads=2, headDim=64)


@pytest.mark.parametrize("bad, code, word", [
    (dict(heads=0), 1, "heads"),
    (dict(kvHeads=3), 1, "kvHeads"),
    (dict(kvHeads=16), 1, "kvHeads"),
    (dict(headDim=0), 1, "headDim"),
    (dict(vHeadDim=-1), 1, "vHeadDim"),
    (dict(posOffset=-1), 1, "posOffset"),
    (dict(window=-1), 1, "window"),
    (dict(window=4, sinks=-1), 1, "sinks"),
    (dict(softcap=-1.0), 1, "softcap"),
    (dict(softcap=float("inf")), 1, "softcap"),
    (dict(softcap=float("nan")), 1, "softcap"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(alibiMax=0.0), 1, "alibiMax"),
    (dict(alibiSlopes=[0.5] * 3), 1, "alibiSlopes"),
    (dict(alibiSlopes=[float("inf")] * 8), 1, "alibiSlopes"),
    (dict(heads=512, kvHeads=512, alibi=True), 2, "attention.alibi"),
])
def test_invalid_params_are_named(bad, code, word):
    kw = dict(BASE)
    kw.update(bad)
    with pytest.raises(ga.AttnError) as ei:
        ga.attn_validate(4, 16, **kw)
    assert ei.value.code == code
    assert word in ei.value.message


def test_negative_sizes_and_bad_bias_kind():
    for T, S in ((-1, 4), (4, -1)):
        with pytest.raises(ga.AttnError) as ei:
            ga.attn_validate(T, S, **BASE)
        assert ei.value.code == 1
    with pytest.raises(ga.AttnError) as ei:
        ga.attn_validate(4, 4, bias_kind=3, **BASE)
    assert "bias" in ei.value.message


def test_valid_params_pass_and_clear_the_error():
    with pytest.raises(ga.AttnError):
        ga.attn_validate(4, 16, heads=0, headDim=8)
    ga.attn_validate(4, 16, **BASE)
    assert ga.attn_last_error() == ""


def test_plans():
    dec = ga.attn_plan(1, 32768, heads=32, kvHeads=8, headDim=128, posOffset=32767)
    assert dec["path"] == "decode" and dec["splits"] > 1
    assert ga.attn_plan(0, 16, **BASE)["path"] == "empty"
    assert ga.attn_plan(4, 0, **BASE)["path"] == "zero"
    # Every row's window lies past the keys: nothing visible, zero fill.
    assert ga.attn_plan(2, 4, posOffset=10, window=2, **BASE)["path"] == "zero"
    # Attention sinks keep keys in view when the window holds none.
    assert ga.attn_plan(2, 4, posOffset=10, window=2, sinks=1, **BASE)["path"] == "decode"
    # Sinks without a window change nothing.
    assert ga.attn_plan(1, 4096, posOffset=4095, sinks=4, **BASE) == ga.attn_plan(1, 4096, posOffset=4095, **BASE)
    # A window that cannot hide any key (causal: wider than the last
    # position; non-causal: at least the largest distance) plans as no window,
    # with or without sinks, however far past 2^31 it reaches.
    dec_kw = dict(heads=32, kvHeads=8, headDim=128, posOffset=32767)
    for w in (32768, 2 ** 31 - 1, 2 ** 40):
        assert ga.attn_plan(1, 32768, window=w, sinks=4, **dec_kw) == ga.attn_plan(1, 32768, **dec_kw)
        assert ga.attn_plan(1024, 1024, causal=False, window=w + 1023 - 32768 if w == 32768 else w,
                            **BASE) == ga.attn_plan(1024, 1024, causal=False, **BASE)
    # One key short of that still takes the windowed plan's sink split.
    assert ga.attn_plan(1, 32768, window=32767, sinks=4, **dec_kw) != ga.attn_plan(1, 32768, **dec_kw)
    # Eight query heads per KV head (64/8, and 28/4 padded to 8) take the
    # decode path at headDim 128: each KV row is read once for the group.
    for H, G in ((64, 8), (28, 4), (8, 1)):
        assert ga.attn_plan(1, 32768, heads=H, kvHeads=G, headDim=128, posOffset=32767)["path"] == "decode"
    # Odd widths have no tuned kernel.
    assert ga.attn_plan(8, 8, heads=4, kvHeads=2, headDim=16)["path"] == "generic"
    assert ga.attn_plan(3, 9, heads=2, headDim=3, vHeadDim=5)["path"] == "generic"


def test_decode_workspace_matches_plan():
    # Room for every split's partial state, plus one more split: the same
    # call made through attn_forward_append may add the split of appended rows.
    kw = dict(heads=32, kvHeads=8, headDim=128, posOffset=32767)
    plan = ga.attn_plan(1, 32768, **kw)
    assert ga.attn_workspace_size(1, 32768, **kw) == 4 * 32 * (plan["splits"] + 1) * (128 + 2)
    assert ga.attn_workspace_size(8, 8, heads=4, kvHeads=2, headDim=16) == 0
    # One split: attn_forward needs none, attn_forward_append may need two.
    short = dict(heads=4, kvHeads=1, headDim=64, posOffset=40)
    assert ga.attn_plan(1, 41, **short)["splits"] == 1
    assert ga.attn_workspace_size(1, 41, **short) == 4 * 4 * 2 * (64 + 2)
    # Relative-position terms: no fused append, no extra split.
    rel = dict(kw, position_bias=dict(weight=4096, buckets=list(range(32))))
    assert ga.attn_workspace_size(1, 32768, **rel) == 4 * 32 * ga.attn_plan(1, 32768, **rel)["splits"] * (128 + 2)


def test_relative_kv_prefill_plans():
    # Relative key/value embeddings on the 32x32x2 prefill kernel: at 128-wide
    # heads the tiles beyond the tables' reach and the band tiles run as two
    # launches, the band one in parts of its own (here 2: 128 workgroups for
    # 256 CUs, (128 + 32) / 32 = 5 band tiles per row block), each leaving a
    # partial state per row; at 64-wide heads one launch covers every tile.
    for D, band in ((128, 2), (64, 0)):
        kw = dict(heads=32, kvHeads=8, headDim=D, posOffset=3584,
                  relative_kv=dict(key=4096, value=8192, max_distance=128))
        plan = ga.attn_plan(512, 4096, **kw)
        assert plan["path"] == "prefill" and plan["variant"] == 32
        try:
            ga.attn_set_option("prefill_splits", 3)
            assert ga.attn_plan(512, 4096, **kw)["splits"] == 3 + band
            assert ga.attn_workspace_size(512, 4096, **kw) == 4 * 512 * 32 * (3 + band) * (D + 2)
            ga.attn_set_option("prefill_splits", 1)
            assert ga.attn_plan(512, 4096, **kw)["splits"] == 1 + band
            assert ga.attn_workspace_size(512, 4096, **kw) == (4 * 512 * 32 * (1 + band) * (D + 2) if band else 0)
        finally:
            ga.attn_set_option("prefill_splits", 0)


@pytest.mark.parametrize("T, H, G, splits", [
    (4096, 32, 8, 1),    # Llama-shaped: 4 heads per workgroup, 128 query blocks per head, 1024 workgroups
    (2048, 32, 8, 2),    # one wave of 512 workgroups for 256 CUs: 1.5 waves (uneven causal blocks)
    (1024, 32, 8, 3),
    (4096, 64, 8, 1),    # 8 heads per KV head in two workgroups of 4
    (4096, 32, 32, 2),   # MHA: 32 query blocks of 128 rows per head, 64 workgroups per XCD
    (2048, 32, 32, 4),
    (8192, 32, 32, 1),
    (4096, 40, 8, 3),    # 5 heads per KV head, one per workgroup: one part more
    (4096, 28, 4, 3),
])
def test_causal_prefill_key_splits(T, H, G, splits):
    # Causal query blocks see unequal key ranges: the planner splits the key
    # ranges to at least 1.5 waves of workgroups and until each head has as
    # many query blocks as an XCD runs workgroups at once.
    plan = ga.attn_plan(T, T, heads=H, kvHeads=G, headDim=128)
    assert plan["path"] == "prefill" and plan["splits"] == splits, plan
    # Non-causal calls give every block the same keys: split only to fill
    # one wave of workgroups (256 of them at 1024 rows: 2 parts).
    nc = ga.attn_plan(T, T, heads=H, kvHeads=G, headDim=128, causal=False)["splits"]
    assert nc == (2 if (T, H, G) == (1024, 32, 8) else 1), nc


@pytest.mark.parametrize("G", [1, 2, 6, 8, 12, 16, 24])
def test_decode_splits_fit_one_wave(G):
    # Two workgroups per CU on 256 CUs: splits x KV groups never passes 512,
    # near and sink splits included.
    kw = dict(heads=G * 2, kvHeads=G, headDim=128, posOffset=65535)
    # (Planning reads no device memory: a stand-in weight address will do.)
    for extra in ({}, dict(window=4096, sinks=4), dict(position_bias=dict(weight=4096, buckets=list(range(32)))),
                  dict(window=4096, sinks=4, position_bias=dict(weight=4096, buckets=list(range(0, 320, 10))))):
        plan = ga.attn_plan(1, 65536, **kw, **extra)
        assert plan["path"] == "decode" and plan["splits"] * G <= 512, (G, extra, plan)
        if "window" not in extra:  # enough keys for most slots (chunks are whole multiples of 64 keys)
            assert plan["splits"] * G > 256, (G, extra, plan)


def test_decode_sink_split():
    # Window 4096 of a 32768-row cache plus 4 sinks: the window splits, then
    # one split of its own for the sink keys below the window.
    # The window takes one split fewer, so the 8 groups' workgroups still fit
    # one wave of 2 per CU.
    kw = dict(heads=32, kvHeads=8, headDim=128, posOffset=32767, window=4096)
    plain = ga.attn_plan(1, 32768, **kw)
    sinks = ga.attn_plan(1, 32768, sinks=4, **kw)
    assert plain["splits"] == 64 and sinks["splits"] == 64
    assert ga.attn_workspace_size(1, 32768, sinks=4, **kw) == 4 * 32 * (sinks["splits"] + 1) * (128 + 2)
    try:
        ga.attn_set_option("decode_splits", 7)
        assert ga.attn_plan(1, 32768, sinks=4, **kw)["splits"] == ga.attn_plan(1, 32768, **kw)["splits"] + 1
    finally:
        ga.attn_set_option("decode_splits", 0)
    # Sinks the window already covers need no split of their own.
    near = dict(kw, posOffset=100)
    assert ga.attn_plan(1, 32768, sinks=4, **near) == ga.attn_plan(1, 32768, **near)


def test_options():
    kw = dict(heads=32, kvHeads=8, headDim=128, posOffset=32767)
    try:
        ga.attn_set_option("decode_splits", 7)
        assert ga.attn_plan(1, 32768, **kw)["splits"] == 7
        ga.attn_set_option("force_path", _lib.ATTN_PATH_GENERIC)
        assert ga.attn_plan(1, 32768, **kw)["path"] == "generic"
    finally:
        ga.attn_set_option("decode_splits", 0)
        ga.attn_set_option("force_path", 0)
    with pytest.raises(ga.AttnError):
        ga.attn_set_option("no_such_option", 1)
    with pytest.raises(ga.AttnError):
        ga.attn_set_option("force_path", 99)


def _forward_raw(p, q, k, v, bias, out, ws=None, ws_bytes=0):
    return _lib.lib().attn_forward(ctypes.byref(p), q, k, v, bias, out, ws, ws_bytes, None)


def test_forward_refuses_before_launch():
    # Fake, never-dereferenced addresses: every case is refused on the host.
    L = _lib.lib()
    p, _ = ga.make_params(4, 16, **BASE)
    A = 1 << 32
    q, k, v, out = A, 2 * A, 3 * A, 4 * A
    assert _forward_raw(p, q, k, v, None, None) == 1 and "out" in ga.attn_last_error()
    assert _forward_raw(p, None, k, v, None, out) == 1 and "q" in ga.attn_last_error()
    assert _forward_raw(p, q, None, v, None, out) == 1 and "k" in ga.attn_last_error()
    assert _forward_raw(p, q, k, v, 5 * A, out) == 1 and "bias" in ga.attn_last_error()
    assert _forward_raw(p, q + 4, k, v, None, out) == 1 and "aligned" in ga.attn_last_error()
    assert _forward_raw(p, q, k, v, None, q + 64) == 1 and "overlaps" in ga.attn_last_error()
    pb, _ = ga.make_params(4, 16, bias_kind=2, **BASE)
    assert _forward_raw(pb, q, k, v, None, out) == 1 and "bias" in ga.attn_last_error()
    # Decode shapes need a workspace.
    pd, _ = ga.make_params(1, 32768, heads=32, kvHeads=8, headDim=128, posOffset=32767)
    assert _forward_raw(pd, q, k, v, None, out) == 1 and "workspace" in ga.attn_last_error()
    assert _forward_raw(pd, q, k, v, None, out, 5 * A + 8, 1 << 30) == 1
    assert "aligned" in ga.attn_last_error()
    # T = 0 is a no-op that succeeds without touching anything.
    p0, _ = ga.make_params(0, 16, **BASE)
    assert _forward_raw(p0, None, None, None, None, None) == 0
    del L


def test_cache_write_refuses_before_launch():
    L = _lib.lib()
    A = 1 << 20
    assert L.attn_cache_write(A, 10, 4, 2 * A, 3, 8, None) == 1
    assert "offset" in ga.attn_last_error()
    assert L.attn_cache_write(A, 10, 4, 2 * A, 1, -1, None) == 1
    assert L.attn_cache_write(A, 10, 0, 2 * A, 1, 0, None) == 1
    assert "width" in ga.attn_last_error()
    assert L.attn_cache_write(A, 10, 4, 2 * A, -1, 0, None) == 1
    assert L.attn_cache_write(None, 10, 4, 2 * A, 1, 0, None) == 1
    assert "cache" in ga.attn_last_error()
    assert L.attn_cache_write(A, 10, 4, A + 16, 2, 1, None) == 1
    assert "overlap" in ga.attn_last_error()
    assert L.attn_cache_write(A, 10, 4, 2 * A, 0, 10, None) == 0  # rows = 0: no-op


def test_cache_write2_refuses_before_launch():
    # Each cache's own checks (named "a: " / "b: "), then the cross checks:
    # neither copy may write rows the other reads or writes. Fake addresses:
    # nothing runs before the checks pass.
    L = _lib.lib()
    A, B = 1 << 20, 1 << 24
    ok = (A, 10, 4, 2 * A, B, 10, 6, 2 * B)
    assert L.attn_cache_write2(*ok, 0, 3, None) == 0  # rows = 0: no-op
    assert L.attn_cache_write2(A, 10, 4, 2 * A, B, 10, 6, 2 * B, 3, 8, None) == 1
    assert ga.attn_last_error().startswith("a: offset")
    assert L.attn_cache_write2(A, 10, 4, 2 * A, B, 4, 6, 2 * B, 2, 3, None) == 1
    assert ga.attn_last_error().startswith("b: offset")
    assert L.attn_cache_write2(A, 10, 4, 2 * A, B, 10, 0, 2 * B, 1, 0, None) == 1
    assert ga.attn_last_error().startswith("b: width")
    assert L.attn_cache_write2(A, 10, 4, 2 * A, None, 10, 6, 2 * B, 1, 0, None) == 1
    assert ga.attn_last_error().startswith("b: cache")
    assert L.attn_cache_write2(A, 10, 4, A + 16, B, 10, 6, 2 * B, 2, 1, None) == 1
    assert ga.attn_last_error().startswith("a: values")
    # b writes rows 1..2 of a cache that starts 16 bytes into a's row 1.
    assert L.attn_cache_write2(A, 10, 4, 2 * A, A + 16, 10, 4, 2 * B, 2, 1, None) == 1
    assert "overlap the rows a writes" in ga.attn_last_error()
    # b reads values that a is writing.
    assert L.attn_cache_write2(A, 10, 4, 2 * A, B, 10, 6, A + 16, 2, 1, None) == 1
    assert "b: values overlap the rows a writes" in ga.attn_last_error()
    assert L.attn_cache_write2(A, 10, 4, B + 48, B, 10, 6, 2 * B, 2, 1, None) == 1
    assert "a: values overlap the rows b writes" in ga.attn_last_error()


def _append_raw(p, q, k, v, k_new, v_new, rows, offset, bias, out, ws=None, ws_bytes=0):
    return _lib.lib().attn_forward_append(ctypes.byref(p), q, k, v, k_new, v_new, rows, offset, bias, out,
                                          ws, ws_bytes, None)


def test_forward_append_refuses_before_launch():
    # Fake, never-dereferenced addresses (caches of 16 rows, 2 KV heads of 64
    # floats: rows of 512 bytes). Every case is refused on the host.
    p, _ = ga.make_params(1, 16, posOffset=15, **BASE)
    A = 1 << 32
    q, k, v, kn, vn, out = A, 2 * A, 3 * A, 4 * A, 5 * A, 6 * A
    assert _append_raw(p, q, k, v, kn, vn, 2, 15, None, out) == 1
    assert ga.attn_last_error().startswith("k: offset")
    assert _append_raw(p, q, k, v, kn, vn, -1, 15, None, out) == 1 and "rows" in ga.attn_last_error()
    assert _append_raw(p, q, k, v, kn, None, 1, 15, None, out) == 1
    assert ga.attn_last_error().startswith("v: values")
    assert _append_raw(p, q, k, v, k + 15 * 512, vn, 1, 15, None, out) == 1
    assert ga.attn_last_error().startswith("k: values")
    # The V rows written start inside the K rows written.
    assert _append_raw(p, q, k, k + 64, kn, vn, 1, 15, None, out) == 1
    assert "overlap the k rows written" in ga.attn_last_error()
    assert _append_raw(p, q, k, v, kn, k + 15 * 512 + 16, 1, 15, None, out) == 1
    assert ga.attn_last_error().startswith("v: values overlap the k rows")
    # q, out, the workspace and the new rows (this call has two splits: it
    # needs a workspace).
    ws = (7 * A, 1 << 20)
    assert _append_raw(p, q, k, v, kn, vn, 1, 15, None, out) == 1 and "workspace" in ga.attn_last_error()
    assert _append_raw(p, k + 15 * 512, k, v, kn, vn, 1, 15, None, out, *ws) == 1
    assert ga.attn_last_error().startswith("q: overlaps the cache rows")
    assert _append_raw(p, q, k, v, kn, vn, 1, 15, None, kn + 64, *ws) == 1
    assert ga.attn_last_error().startswith("out: overlaps k_new")
    assert _append_raw(p, q, k, v, kn, vn, 1, 15, None, out, vn - 256, 1 << 20) == 1
    assert ga.attn_last_error().startswith("workspace: overlaps k_new")
    # attn_forward's own checks still apply.
    assert _append_raw(p, None, k, v, kn, vn, 1, 15, None, out) == 1 and "q" in ga.attn_last_error()
    assert _append_raw(p, q, k, v, kn, vn, 1, 15, None, out + 4) == 1 and "aligned" in ga.attn_last_error()
    pd, _ = ga.make_params(1, 32768, heads=32, kvHeads=8, headDim=128, posOffset=32767)
    assert _append_raw(pd, q, k, v, kn, vn, 1, 32767, None, out) == 1 and "workspace" in ga.attn_last_error()
    # T = 0 and no rows: nothing to do.
    p0, _ = ga.make_params(0, 16, **BASE)
    assert _append_raw(p0, None, None, None, None, None, 0, 0, None, None) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 64)
    with pytest.raises(ValueError):
        ga.attn_forward(q, q, q, heads=1, headDim=64)
    with pytest.raises(ValueError):
        ga.attn_forward_append(q, q, q, q, q, 0, heads=1, headDim=64)


MLA = dict(heads=16, kv_rank=512, qk_nope=128, qk_rope=64, v_head_dim=128)


@pytest.mark.parametrize("bad, code, word", [
    (dict(heads=0), 1, "heads"),
    (dict(kv_rank=0), 1, "kv_rank"),
    (dict(qk_nope=0), 1, "qk_nope"),
    (dict(qk_rope=-1), 1, "qk_rope"),
    (dict(v_head_dim=0), 1, "v_head_dim"),
    (dict(posOffset=-1), 1, "posOffset"),
    (dict(window=-2), 1, "window"),
    (dict(window=4, sinks=-1), 1, "sinks"),
    (dict(scale=float("inf")), 1, "scale"),
    (dict(kv_rank=12000, qk_rope=8), 2, "kv_rank"),
])
def test_mla_invalid_params_are_named(bad, code, word):
    kw = dict(MLA)
    kw.update(bad)
    with pytest.raises(ga.AttnError) as ei:
        ga.attn_mla_validate(1, 64, **kw)
    assert ei.value.code == code
    assert word in ei.value.message


def test_mla_plans_and_workspace():
    dec = ga.attn_mla_plan(1, 8192, posOffset=8191, **MLA)
    assert dec["path"] == "mla" and dec["tile_q"] == 16 and dec["splits"] > 1 and dec["slices"] == 8
    # q_abs (16 rows x 576 floats, 256-byte aligned), the splits' partial
    # states (256-byte aligned), then each row's 8 slice shares of the 128
    # outputs (256-byte aligned) and one counter per row.
    a256 = lambda n: -(-n // 256) * 256
    part = a256(16 * dec["splits"] * (512 + 2) * 4)
    want = 16 * 576 * 4 + part + a256(16 * 8 * 128 * 4) + 16 * 4
    assert ga.attn_mla_workspace_size(1, 8192, posOffset=8191, **MLA) == want
    try:
        ga.attn_set_option("mla_slices", -1)
        assert ga.attn_mla_plan(1, 8192, posOffset=8191, **MLA)["slices"] == 0
        assert ga.attn_mla_workspace_size(1, 8192, posOffset=8191, **MLA) == 16 * 576 * 4 + part
    finally:
        ga.attn_set_option("mla_slices", 0)
    # v_head_dim past 256 keeps the per-output merge.
    assert ga.attn_mla_plan(1, 8192, posOffset=8191, **dict(MLA, v_head_dim=320))["slices"] == 0
    with pytest.raises(ga.AttnError):
        ga.attn_set_option("mla_slices", 2)
    assert ga.attn_mla_plan(0, 16, **MLA)["path"] == "empty"
    assert ga.attn_mla_plan(1, 0, **MLA)["path"] == "zero"
    assert ga.attn_mla_workspace_size(1, 0, **MLA) == 0
    # Shapes without a matrix-core instance take the generic kernel, one split.
    gen = ga.attn_mla_plan(2, 50, heads=3, kv_rank=48, qk_nope=8, qk_rope=16, v_head_dim=8)
    assert gen["path"] == "mla" and gen["tile_q"] == 1 and gen["splits"] == 1 and gen["slices"] == 0
    # The sink keys below a window take a split of their own.
    kw = dict(MLA, posOffset=8191, window=1024)
    assert ga.attn_mla_plan(1, 8192, sinks=4, **kw)["splits"] == ga.attn_mla_plan(1, 8192, **kw)["splits"] + 1
    try:
        ga.attn_set_option("mla_splits", 5)
        assert ga.attn_mla_plan(1, 8192, posOffset=8191, **MLA)["splits"] == 5
        ga.attn_set_option("mla_generic", 1)
        assert ga.attn_mla_plan(1, 8192, posOffset=8191, **MLA)["tile_q"] == 1
    finally:
        ga.attn_set_option("mla_splits", 0)
        ga.attn_set_option("mla_generic", 0)
    with pytest.raises(ga.AttnError):
        ga.attn_set_option("mla_generic", 2)
