"""Python binding of libattn.so, with the C ABI's names.

Argument marshalling only: every step of the op runs in the library's HIP
kernels. PyTorch supplies device memory (the output and workspace tensors)
and the current stream. Parameters take the op catalogue's names for the
`attention` op (heads, headDim, kvHeads, vHeadDim, causal, posOffset, scale,
softcap, window, alibi, alibiMax, alibiSlopes) and the `rope` op (headDim,
base, offset, rotaryDim, interleaved, scaling, invFreq, attentionFactor).
"""

from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence

from . import _lib
from ._lib import AttnParams, AttnPlanInfo, AttnRopeParams


class AttnError(RuntimeError):
    """A call the library refused (code and message from attn_last_error)."""

    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


def attn_last_error() -> str:
    return _lib.lib().attn_last_error().decode()


def _check(rc: int) -> None:
    if rc != _lib.ATTN_OK:
        raise AttnError(rc, attn_last_error())


def make_rope_params(headDim: Optional[int] = None, base: Optional[float] = None,
                     offset: Optional[int] = None, rotaryDim: Optional[int] = None,
                     interleaved: Optional[bool] = None, scaling: Optional[dict] = None,
                     invFreq: Optional[Sequence[float]] = None,
                     attentionFactor: Optional[float] = None):
    """attn_rope_params for one call. `scaling` is a model config's rope_scaling
    object as it stands (its rope_type or type, factor, low_freq_factor,
    high_freq_factor, original_max_position_embeddings, max_position_embeddings,
    beta_fast, beta_slow, mscale, mscale_all_dim, truncate, short_factor,
    long_factor, attention_factor). Returns (params, keepalive)."""
    L = _lib.lib()
    r = AttnRopeParams()
    L.attn_rope_params_init(ctypes.byref(r))
    r.head_dim = int(headDim or 0)
    r.rotary_dim = int(rotaryDim or 0)
    r.offset = int(offset or 0)
    r.interleaved = 1 if interleaved else 0
    if base is not None:
        r.base = float(base)
    half = (r.rotary_dim or r.head_dim) // 2
    keep = []

    def doubles(name, values):
        if len(values) != half:
            raise AttnError(_lib.ATTN_ERR_INVALID, f"rope.scaling: {name} holds {len(values)} values, "
                            f"rotaryDim/2 = {half} expected")
        arr = (ctypes.c_double * half)(*[float(x) for x in values])
        keep.append(arr)
        return ctypes.cast(arr, ctypes.POINTER(ctypes.c_double))

    if invFreq is not None:
        if len(invFreq) != half:
            raise AttnError(_lib.ATTN_ERR_INVALID, f"rope.invFreq: {len(invFreq)} values, "
                            f"rotaryDim/2 = {half} expected")
        import numpy as np
        arr = (ctypes.c_float * half)(*np.asarray(invFreq, dtype=np.float64).astype(np.float32).tolist())
        keep.append(arr)
        r.inv_freq = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    if attentionFactor is not None:
        r.has_attention_factor, r.attention_factor = 1, float(attentionFactor)
    if scaling:
        kind = scaling.get("rope_type", scaling.get("type"))
        if kind not in _lib.ROPE_SCALING:
            raise AttnError(_lib.ATTN_ERR_UNSUPPORTED, f"rope.scaling: unknown type {kind!r}")
        r.scaling = _lib.ROPE_SCALING[kind]
        num = {"factor": "factor", "low_freq_factor": "low_freq_factor",
               "high_freq_factor": "high_freq_factor", "beta_fast": "beta_fast",
               "beta_slow": "beta_slow", "mscale": "mscale", "mscale_all_dim": "mscale_all_dim",
               "attention_factor": "scaling_attention_factor"}
        for key, field in num.items():
            if scaling.get(key) is not None:
                setattr(r, field, float(scaling[key]))
        if scaling.get("original_max_position_embeddings") is not None:
            r.original_max_positions = int(scaling["original_max_position_embeddings"])
        if scaling.get("max_position_embeddings") is not None:
            r.max_positions = int(scaling["max_position_embeddings"])
        if scaling.get("truncate") is not None:
            r.truncate = 1 if scaling["truncate"] else 0
        if scaling.get("short_factor") is not None:
            r.short_factor = doubles("short_factor", scaling["short_factor"])
        if scaling.get("long_factor") is not None:
            r.long_factor = doubles("long_factor", scaling["long_factor"])
    return r, keep


def make_params(T: int, S: int, *, heads: int, headDim: int, kvHeads: Optional[int] = None,
                vHeadDim: Optional[int] = None, causal: Optional[bool] = None,
                posOffset: Optional[int] = None, scale: Optional[float] = None,
                softcap: Optional[float] = None, window: Optional[int] = None,
                alibi: Optional[bool] = None, alibiMax: Optional[float] = None,
                alibiSlopes: Optional[Sequence[float]] = None, bias_kind: int = 0,
                q_rope: Optional[dict] = None, sinks: Optional[int] = None,
                position_bias: Optional[dict] = None, relative_kv: Optional[dict] = None):
    """attn_params for one call. Returns (params, keepalive) - keep the second
    alive until the call returns (it owns the explicit slope array and the
    q_rope parameters). q_rope holds `rope` op params for q; its headDim
    defaults to headDim and its offset to posOffset. sinks: attention sinks
    beside the window (keys s < sinks stay visible). position_bias: {weight,
    buckets, bidirectional} (weight a GPU tensor [n or 2n, heads], buckets
    the n ascending distance thresholds). relative_kv: {key, value,
    max_distance} (GPU tensors [2*max_distance+1, headDim / vHeadDim])."""
    L = _lib.lib()
    p = AttnParams()
    L.attn_params_init(ctypes.byref(p))
    p.T, p.S = int(T), int(S)
    p.heads, p.head_dim = int(heads), int(headDim)
    p.kv_heads = int(kvHeads) if kvHeads else 0
    p.v_head_dim = int(vHeadDim) if vHeadDim else 0
    if causal is not None:
        p.causal = 1 if causal else 0
    if posOffset is not None:
        p.pos_offset = int(posOffset)
    if scale is not None:
        p.has_scale, p.scale = 1, float(scale)
    if softcap is not None:
        p.softcap = float(softcap)
    if window is not None:
        p.window = int(window)
    if sinks is not None:
        p.sinks = int(sinks)
    extra = []
    if position_bias is not None:
        buckets = [int(b) for b in position_bias["buckets"]]
        arr = (ctypes.c_int64 * max(1, len(buckets)))(*buckets)
        extra.append(arr)
        p.pb_weight = _ptr(position_bias["weight"])
        p.pb_buckets = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64))
        p.pb_n = len(buckets)
        p.pb_bidirectional = 1 if position_bias.get("bidirectional") else 0
    if relative_kv is not None:
        p.rel_k = _ptr(relative_kv["key"])
        p.rel_v = _ptr(relative_kv.get("value"))
        p.rel_max = int(relative_kv["max_distance"])
    keep = None
    if alibiSlopes is not None:
        # The C ABI takes `heads` floats; only the caller knows the list's length.
        if len(alibiSlopes) != int(heads):
            raise AttnError(_lib.ATTN_ERR_INVALID,
                            f"alibiSlopes: {len(alibiSlopes)} slopes for {heads} heads")
        keep = (ctypes.c_float * len(alibiSlopes))(*[float(x) for x in alibiSlopes])
        p.alibi = _lib.ATTN_ALIBI_EXPLICIT
        p.alibi_slopes = ctypes.cast(keep, ctypes.POINTER(ctypes.c_float))
    elif alibiMax is not None:
        p.alibi, p.alibi_max = _lib.ATTN_ALIBI_MPT, float(alibiMax)
    elif alibi:
        p.alibi = _lib.ATTN_ALIBI_BLOOM
    p.bias_kind = int(bias_kind)
    if q_rope is not None:
        rp = dict(q_rope)
        rp.setdefault("headDim", headDim)
        if rp.get("offset") is None:
            rp["offset"] = posOffset or 0
        r, rkeep = make_rope_params(**rp)
        keep = (keep, r, rkeep)
        p.q_rope = ctypes.pointer(r)
    if extra:
        keep = (keep, extra)
    return p, keep


def _ptr(x):
    """Device address of a tensor argument inside the params (None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def attn_validate(T: int, S: int, bias_kind: int = 0, **params) -> None:
    p, keep = make_params(T, S, bias_kind=bias_kind, **params)
    _check(_lib.lib().attn_validate(ctypes.byref(p)))
    del keep


def attn_workspace_size(T: int, S: int, bias_kind: int = 0, **params) -> int:
    p, keep = make_params(T, S, bias_kind=bias_kind, **params)
    n = _lib.lib().attn_workspace_size(ctypes.byref(p))
    del keep
    return int(n)


def attn_plan(T: int, S: int, bias_kind: int = 0, **params) -> dict:
    p, keep = make_params(T, S, bias_kind=bias_kind, **params)
    info = AttnPlanInfo()
    _check(_lib.lib().attn_plan(ctypes.byref(p), ctypes.byref(info)))
    del keep
    return {"path": _lib.PATH_NAMES.get(info.path, str(info.path)), "splits": info.splits,
            "tile_q": info.tile_q, "variant": info.variant}


def attn_set_option(name: str, value: int) -> None:
    _check(_lib.lib().attn_set_option(name.encode(), int(value)))


def attn_timing_enable(on: bool) -> None:
    _check(_lib.lib().attn_timing_enable(1 if on else 0))


def attn_timing_collect(kernel: str):
    """(total milliseconds, launches) for `kernel` since the last collect."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(_lib.lib().attn_timing_collect(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


# -- device calls --------------------------------------------------------------

_workspaces = {}


def _torch():
    import torch
    return torch


def _dev_tensor(x, name: str):
    torch = _torch()
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor (got {x.device})")
    if x.dtype != torch.float32:
        raise ValueError(f"{name}: must be float32 (got {x.dtype})")
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous row-major")
    return x


def _stream_ptr(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_for(nbytes: int, device, stream=None):
    """A cached device buffer of at least nbytes (None for 0), one per
    (device, stream): calls in flight at the same time must not share a
    workspace, and calls on one stream run in order. The buffer is allocated
    with its stream current, so when a larger one replaces it the caching
    allocator hands the old memory out again only in that stream's order."""
    if nbytes <= 0:
        return None
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    key = (device.type, device.index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(stream):
            ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _check_forward(q, k, v, bias, out, params):
    """Shape, dtype and device checks; returns (T, S, heads, vHeadDim, bias_kind)."""
    _dev_tensor(q, "q")
    _dev_tensor(k, "k")
    _dev_tensor(v, "v")
    if q.dim() != 2 or k.dim() != 2 or v.dim() != 2:
        raise ValueError("q, k and v are flat 2-D tensors [rows, heads*width]")
    T, S = q.shape[0], k.shape[0]
    H = int(params["heads"])
    D = int(params["headDim"])
    G = int(params.get("kvHeads") or H)
    Dv = int(params.get("vHeadDim") or D)
    if q.shape[1] != H * D:
        raise ValueError(f"q: {tuple(q.shape)} is not [T, heads*headDim] = [T, {H * D}]")
    if k.shape[1] != G * D:
        raise ValueError(f"k: {tuple(k.shape)} is not [S, kvHeads*headDim] = [S, {G * D}]")
    if tuple(v.shape) != (S, G * Dv):
        raise ValueError(f"v: {tuple(v.shape)} is not [S, kvHeads*vHeadDim] = [{S}, {G * Dv}]")
    bias_kind = _lib.ATTN_BIAS_NONE
    if bias is not None:
        _dev_tensor(bias, "bias")
        if tuple(bias.shape) == (T, S):
            bias_kind = _lib.ATTN_BIAS_TS
        elif tuple(bias.shape) == (H, T, S):
            bias_kind = _lib.ATTN_BIAS_HTS
        else:
            raise ValueError(f"bias: {tuple(bias.shape)} is neither [T, S] nor [heads, T, S]")
    if out is not None:
        _dev_tensor(out, "out")
        if tuple(out.shape) != (T, H * Dv):
            raise ValueError(f"out: {tuple(out.shape)} is not [T, heads*vHeadDim] = [{T}, {H * Dv}]")
    pb = params.get("position_bias")
    if pb is not None:
        _dev_tensor(pb["weight"], "position_bias.weight")
        n = len(pb["buckets"]) * (2 if pb.get("bidirectional") else 1)
        if tuple(pb["weight"].shape) != (n, H):
            raise ValueError(f"position_bias.weight: {tuple(pb['weight'].shape)} is not [{n}, heads={H}]")
    rk = params.get("relative_kv")
    if rk is not None:
        m = int(rk["max_distance"])
        _dev_tensor(rk["key"], "relative_kv.key")
        if tuple(rk["key"].shape) != (2 * m + 1, D):
            raise ValueError(f"relative_kv.key: {tuple(rk['key'].shape)} is not [{2 * m + 1}, headDim={D}]")
        if rk.get("value") is not None:
            _dev_tensor(rk["value"], "relative_kv.value")
            if tuple(rk["value"].shape) != (2 * m + 1, Dv):
                raise ValueError(f"relative_kv.value: {tuple(rk['value'].shape)} is not [{2 * m + 1}, vHeadDim={Dv}]")
    return T, S, H, Dv, bias_kind


def attn_forward(q, k, v, bias=None, *, out=None, workspace=None, stream=None, **params):
    """Op `attention`: returns out [T, heads*vHeadDim] (float32, on q's device).

    q [T, heads*headDim], k [S, kvHeads*headDim], v [S, kvHeads*vHeadDim] and the
    optional bias [T, S] or [heads, T, S] are contiguous float32 GPU tensors.
    """
    torch = _torch()
    T, S, H, Dv, bias_kind = _check_forward(q, k, v, bias, out, params)
    p, keep = make_params(T, S, bias_kind=bias_kind, **params)
    L = _lib.lib()
    if out is None:
        out = torch.empty((T, H * Dv), dtype=torch.float32, device=q.device)
    need = int(L.attn_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = workspace_for(need, q.device, stream)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = L.attn_forward(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                        bias.data_ptr() if bias is not None else None, out.data_ptr(),
                        ws_ptr, ws_bytes, _stream_ptr(stream, q.device))
    del keep
    _check(rc)
    return out


def attn_forward_noalloc(q, k, v, bias=None, *, out, stream=None, **params):
    """attn_forward with the split state in the library's own per-GPU scratch
    array: the call allocates nothing, so `out` [T, heads*vHeadDim] must be
    given. Calls that overlap in time on one GPU race on that array. Returns out."""
    T, S, H, Dv, bias_kind = _check_forward(q, k, v, bias, out, params)
    p, keep = make_params(T, S, bias_kind=bias_kind, **params)
    rc = _lib.lib().attn_forward_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                         bias.data_ptr() if bias is not None else None, out.data_ptr(),
                                         _stream_ptr(stream, q.device))
    del keep
    _check(rc)
    return out


def prepare_forward(q, k, v, bias=None, *, out, workspace=None, stream=None, **params):
    """Marshal one attn_forward call once and return a zero-argument callable
    that repeats it (same tensors, same stream). For timing loops, where
    rebuilding the ctypes arguments on every call would cost more host time
    than the kernels take. The tensors must outlive the callable."""
    T, S, _, _, bias_kind = _check_forward(q, k, v, bias, out, params)
    p, keep = make_params(T, S, bias_kind=bias_kind, **params)
    L = _lib.lib()
    need = int(L.attn_workspace_size(ctypes.byref(p)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = workspace_for(need, q.device, stream)
    args = (ctypes.byref(p), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
            ctypes.c_void_p(v.data_ptr()),
            ctypes.c_void_p(bias.data_ptr() if bias is not None else None),
            ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(workspace.data_ptr() if workspace is not None else None),
            ctypes.c_size_t(workspace.numel() * workspace.element_size() if workspace is not None else 0),
            _stream_ptr(stream, q.device))
    fn = L.attn_forward
    held = (p, keep, q, k, v, bias, out, workspace)

    def call():
        rc = fn(*args)
        if rc != _lib.ATTN_OK:
            raise AttnError(rc, attn_last_error())

    call.held = held
    return call


def _forward_append_args(q, k, v, k_new, v_new, offset, bias, out, workspace, stream, params):
    torch = _torch()
    T, S, H, Dv, bias_kind = _check_forward(q, k, v, bias, out, params)
    _dev_tensor(k_new, "k_new")
    _dev_tensor(v_new, "v_new")
    if k_new.dim() != 2 or k_new.shape[1] != k.shape[1]:
        raise ValueError(f"k_new: {tuple(k_new.shape)} is not [rows, kvHeads*headDim = {k.shape[1]}]")
    if tuple(v_new.shape) != (k_new.shape[0], v.shape[1]):
        raise ValueError(f"v_new: {tuple(v_new.shape)} is not [rows = {k_new.shape[0]}, {v.shape[1]}]")
    p, keep = make_params(T, S, bias_kind=bias_kind, **params)
    L = _lib.lib()
    if out is None:
        out = torch.empty((T, H * Dv), dtype=torch.float32, device=q.device)
    need = int(L.attn_workspace_size(ctypes.byref(p)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = workspace_for(need, q.device, stream)
    args = (ctypes.byref(p), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
            ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(k_new.data_ptr()),
            ctypes.c_void_p(v_new.data_ptr()), ctypes.c_int64(k_new.shape[0]), ctypes.c_int64(int(offset)),
            ctypes.c_void_p(bias.data_ptr() if bias is not None else None),
            ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(workspace.data_ptr() if workspace is not None else None),
            ctypes.c_size_t(workspace.numel() * workspace.element_size() if workspace is not None else 0),
            _stream_ptr(stream, q.device))
    return args, (p, keep, q, k, v, k_new, v_new, bias, out, workspace), out


def attn_forward_append(q, k, v, k_new, v_new, offset: int, bias=None, *, out=None, workspace=None,
                        stream=None, **params):
    """A decode step in one call: rows [offset, offset + rows) of the caches k
    and v become k_new and v_new [rows, ...] (op `cache_write`), then op
    `attention` of q over the caches. Returns out [T, heads*vHeadDim]."""
    args, held, out = _forward_append_args(q, k, v, k_new, v_new, offset, bias, out, workspace, stream, params)
    rc = _lib.lib().attn_forward_append(*args)
    del held
    _check(rc)
    return out


def prepare_forward_append(q, k, v, k_new, v_new, offset: int, bias=None, *, out, workspace=None, stream=None,
                           **params):
    """Like prepare_forward, for attn_forward_append."""
    args, held, _ = _forward_append_args(q, k, v, k_new, v_new, offset, bias, out, workspace, stream, params)
    fn = _lib.lib().attn_forward_append

    def call():
        rc = fn(*args)
        if rc != _lib.ATTN_OK:
            raise AttnError(rc, attn_last_error())

    call.held = held
    return call


def prepare_cache_write(cache, values, offset: int, *, stream=None):
    """Like prepare_forward, for attn_cache_write."""
    _dev_tensor(cache, "cache")
    _dev_tensor(values, "values")
    args = (ctypes.c_void_p(cache.data_ptr()), ctypes.c_int64(cache.shape[0]),
            ctypes.c_int64(cache.shape[1]), ctypes.c_void_p(values.data_ptr()),
            ctypes.c_int64(values.shape[0]), ctypes.c_int64(int(offset)),
            _stream_ptr(stream, cache.device))
    fn = _lib.lib().attn_cache_write
    held = (cache, values)

    def call():
        rc = fn(*args)
        if rc != _lib.ATTN_OK:
            raise AttnError(rc, attn_last_error())

    call.held = held
    return call


def attn_cache_write(cache, values, offset: int, *, stream=None):
    """Op `cache_write`: rows [offset, offset+rows) of `cache` become `values`, in place.
    Returns the cache."""
    _dev_tensor(cache, "cache")
    _dev_tensor(values, "values")
    if cache.dim() != 2 or values.dim() != 2 or cache.shape[1] != values.shape[1]:
        raise ValueError("cache [maxRows, width] and values [rows, width] must share width")
    rc = _lib.lib().attn_cache_write(cache.data_ptr(), cache.shape[0], cache.shape[1],
                                     values.data_ptr(), values.shape[0], int(offset),
                                     _stream_ptr(stream, cache.device))
    _check(rc)
    return cache


def _cache_write2_args(cache_a, values_a, cache_b, values_b, offset, stream):
    for t, n in ((cache_a, "cache_a"), (values_a, "values_a"), (cache_b, "cache_b"), (values_b, "values_b")):
        _dev_tensor(t, n)
    for c, v in ((cache_a, values_a), (cache_b, values_b)):
        if c.dim() != 2 or v.dim() != 2 or c.shape[1] != v.shape[1]:
            raise ValueError("each cache [maxRows, width] and its values [rows, width] must share width")
    if values_a.shape[0] != values_b.shape[0]:
        raise ValueError("values_a and values_b must hold the same number of rows")
    return (ctypes.c_void_p(cache_a.data_ptr()), ctypes.c_int64(cache_a.shape[0]), ctypes.c_int64(cache_a.shape[1]),
            ctypes.c_void_p(values_a.data_ptr()),
            ctypes.c_void_p(cache_b.data_ptr()), ctypes.c_int64(cache_b.shape[0]), ctypes.c_int64(cache_b.shape[1]),
            ctypes.c_void_p(values_b.data_ptr()),
            ctypes.c_int64(values_a.shape[0]), ctypes.c_int64(int(offset)), _stream_ptr(stream, cache_a.device))


def attn_cache_write2(cache_a, values_a, cache_b, values_b, offset: int, *, stream=None):
    """Two `cache_write` ops at the same rows in one launch (a decode step's new
    K and V rows). Returns (cache_a, cache_b)."""
    _check(_lib.lib().attn_cache_write2(*_cache_write2_args(cache_a, values_a, cache_b, values_b, offset, stream)))
    return cache_a, cache_b


def prepare_cache_write2(cache_a, values_a, cache_b, values_b, offset: int, *, stream=None):
    """Like prepare_forward, for attn_cache_write2."""
    args = _cache_write2_args(cache_a, values_a, cache_b, values_b, offset, stream)
    fn = _lib.lib().attn_cache_write2
    held = (cache_a, values_a, cache_b, values_b)

    def call():
        rc = fn(*args)
        if rc != _lib.ATTN_OK:
            raise AttnError(rc, attn_last_error())

    call.held = held
    return call


# -- op `rope` -------------------------------------------------------------------

def attn_rope_table(rows: int = 1, **rope):
    """(inverse frequencies as a float32 numpy array, attention factor) that the
    library uses for `rows` rows starting at rope's offset."""
    import numpy as np
    r, keep = make_rope_params(**rope)
    half = (r.rotary_dim or r.head_dim) // 2
    buf = (ctypes.c_float * max(half, 1))()
    af = ctypes.c_float()
    _check(_lib.lib().attn_rope_table(ctypes.byref(r), int(rows), buf, ctypes.byref(af)))
    del keep
    return np.ctypeslib.as_array(buf)[:half].copy(), float(af.value)


def attn_rope(x, *, out=None, stream=None, **rope):
    """Op `rope` on x [T, heads*headDim]; out may be x itself (in place)."""
    torch = _torch()
    _dev_tensor(x, "x")
    if x.dim() != 2:
        raise ValueError("x: must be [T, heads*headDim]")
    if out is None:
        out = torch.empty_like(x)
    _dev_tensor(out, "out")
    if tuple(out.shape) != tuple(x.shape):
        raise ValueError("out: must have the shape of x")
    r, keep = make_rope_params(**rope)
    rc = _lib.lib().attn_rope(ctypes.byref(r), x.shape[0], x.shape[1], x.data_ptr(), out.data_ptr(),
                              _stream_ptr(stream, x.device))
    del keep
    _check(rc)
    return out


def _rope_cache_args(cache, values, offset, stream, rope):
    _dev_tensor(cache, "cache")
    _dev_tensor(values, "values")
    if cache.dim() != 2 or values.dim() != 2 or cache.shape[1] != values.shape[1]:
        raise ValueError("cache [maxRows, width] and values [rows, width] must share width")
    rope = dict(rope)
    if rope.get("offset") is None:
        rope["offset"] = int(offset)
    r, keep = make_rope_params(**rope)
    args = (ctypes.c_void_p(cache.data_ptr()), ctypes.c_int64(cache.shape[0]),
            ctypes.c_int64(cache.shape[1]), ctypes.c_void_p(values.data_ptr()),
            ctypes.c_int64(values.shape[0]), ctypes.c_int64(int(offset)), ctypes.byref(r),
            _stream_ptr(stream, cache.device))
    return args, (r, keep, cache, values)


def attn_rope_cache_write(cache, values, offset: int, rope: dict, *, stream=None):
    """Ops `rope` then `cache_write`: rows [offset, offset+rows) of `cache` become
    rope(values), in place. `rope` holds the rope op's params; the rows'
    positions start at its offset, which defaults to the cache offset.
    Returns the cache."""
    args, held = _rope_cache_args(cache, values, offset, stream, rope)
    rc = _lib.lib().attn_rope_cache_write(*args)
    del held
    _check(rc)
    return cache


def prepare_rope_cache_write(cache, values, offset: int, rope: dict, *, stream=None):
    """Like prepare_forward, for attn_rope_cache_write."""
    args, held = _rope_cache_args(cache, values, offset, stream, rope)
    fn = _lib.lib().attn_rope_cache_write

    def call():
        rc = fn(*args)
        if rc != _lib.ATTN_OK:
            raise AttnError(rc, attn_last_error())

    call.held = held
    return call


# -- latent (MLA) attention ----------------------------------------------------

def make_mla_params(T: int, S: int, *, heads: int, kv_rank: int, qk_nope: int, qk_rope: int,
                    v_head_dim: int, scale: Optional[float] = None, causal: Optional[bool] = None,
                    posOffset: Optional[int] = None, window: Optional[int] = None,
                    sinks: Optional[int] = None):
    """attn_mla_params for one call (the IR schema's op_mla_attention names,
    plus posOffset)."""
    p = _lib.AttnMlaParams()
    _lib.lib().attn_mla_params_init(ctypes.byref(p))
    p.T, p.S = int(T), int(S)
    p.heads, p.kv_rank, p.qk_nope = int(heads), int(kv_rank), int(qk_nope)
    p.qk_rope, p.v_head_dim = int(qk_rope), int(v_head_dim)
    if causal is not None:
        p.causal = 1 if causal else 0
    if posOffset is not None:
        p.pos_offset = int(posOffset)
    if scale is not None:
        p.has_scale, p.scale = 1, float(scale)
    if window is not None:
        p.window = int(window)
    if sinks is not None:
        p.sinks = int(sinks)
    return p


def attn_mla_validate(T: int, S: int, **params) -> None:
    p = make_mla_params(T, S, **params)
    _check(_lib.lib().attn_mla_validate(ctypes.byref(p)))


def attn_mla_workspace_size(T: int, S: int, **params) -> int:
    p = make_mla_params(T, S, **params)
    return int(_lib.lib().attn_mla_workspace_size(ctypes.byref(p)))


def attn_mla_plan(T: int, S: int, **params) -> dict:
    p = make_mla_params(T, S, **params)
    info = AttnPlanInfo()
    _check(_lib.lib().attn_mla_plan(ctypes.byref(p), ctypes.byref(info)))
    return {"path": _lib.PATH_NAMES.get(info.path, str(info.path)), "splits": info.splits,
            "tile_q": info.tile_q, "slices": info.variant}


def _check_mla(q, state, k_b, v_b, out, params):
    for x, name in ((q, "q"), (state, "state"), (k_b, "k_b"), (v_b, "v_b")):
        _dev_tensor(x, name)
    H, R, N = int(params["heads"]), int(params["kv_rank"]), int(params["qk_nope"])
    P, Dv = int(params["qk_rope"]), int(params["v_head_dim"])
    if q.dim() != 2 or q.shape[1] != H * (N + P):
        raise ValueError(f"q: {tuple(q.shape)} is not [T, heads*(qk_nope+qk_rope)] = [T, {H * (N + P)}]")
    if state.dim() != 2 or state.shape[1] != R + P:
        raise ValueError(f"state: {tuple(state.shape)} is not [S, kv_rank+qk_rope] = [S, {R + P}]")
    if tuple(k_b.shape) != (H, N, R):
        raise ValueError(f"k_b: {tuple(k_b.shape)} is not [heads, qk_nope, kv_rank] = {(H, N, R)}")
    if tuple(v_b.shape) != (H, Dv, R):
        raise ValueError(f"v_b: {tuple(v_b.shape)} is not [heads, v_head_dim, kv_rank] = {(H, Dv, R)}")
    T = q.shape[0]
    if out is not None:
        _dev_tensor(out, "out")
        if tuple(out.shape) != (T, H * Dv):
            raise ValueError(f"out: {tuple(out.shape)} is not [T, heads*v_head_dim] = [{T}, {H * Dv}]")
    return T, state.shape[0], H, Dv


def _mla_args(q, state, k_b, v_b, out, workspace, stream, params):
    T, S, H, Dv = _check_mla(q, state, k_b, v_b, out, params)
    p = make_mla_params(T, S, **params)
    L = _lib.lib()
    if out is None:
        out = _torch().empty((T, H * Dv), dtype=_torch().float32, device=q.device)
    need = int(L.attn_mla_workspace_size(ctypes.byref(p)))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = workspace_for(need, q.device, stream)
    args = (ctypes.byref(p), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(state.data_ptr()),
            ctypes.c_void_p(k_b.data_ptr()), ctypes.c_void_p(v_b.data_ptr()), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(workspace.data_ptr() if workspace is not None else None),
            ctypes.c_size_t(workspace.numel() * workspace.element_size() if workspace is not None else 0),
            _stream_ptr(stream, q.device))
    return args, (p, q, state, k_b, v_b, out, workspace), out


def attn_mla_forward(q, state, k_b, v_b, *, out=None, workspace=None, stream=None, **params):
    """Latent (MLA) attention: returns out [T, heads*v_head_dim] (float32).

    q [T, heads*(qk_nope+qk_rope)], state [S, kv_rank+qk_rope], k_b [heads,
    qk_nope, kv_rank] and v_b [heads, v_head_dim, kv_rank] are contiguous
    float32 GPU tensors."""
    args, held, out = _mla_args(q, state, k_b, v_b, out, workspace, stream, params)
    rc = _lib.lib().attn_mla_forward(*args)
    del held
    _check(rc)
    return out


def prepare_mla_forward(q, state, k_b, v_b, *, out, workspace=None, stream=None, **params):
    """Marshal one attn_mla_forward call once; returns a callable repeating it."""
    args, held, _ = _mla_args(q, state, k_b, v_b, out, workspace, stream, params)
    fn = _lib.lib().attn_mla_forward

    def call():
        rc = fn(*args)
        if rc != _lib.ATTN_OK:
            raise AttnError(rc, attn_last_error())

    call.held = held
    return call
