"""Attention oracle (test infrastructure only).

A plain, slow CPU definition of the graph protocol's `attention` and
`cache_write` ops, used to check the HIP library. Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import this package; the
library never does, and the two share no code. The only thing both sides
take from elsewhere is their seeded input arrays.

Parameter handling follows the op catalogue's `attention` entry (graph
protocol op catalogue, op `attention`, params):

* kvHeads defaults to heads; query head h reads key/value head
  floor(h * kvHeads / heads) (contiguous groups, the usual grouped-query
  layout; the page names grouped-query support and gives no mapping).
* vHeadDim defaults to headDim.
* causal defaults to true; posOffset defaults to 0 and key row s sits at
  absolute position s.
* scale defaults to 1/sqrt(headDim), which is what it "replaces".
* softcap and window: absent or 0 means off; negative values are refused.
* sinks (not a catalogue param: the IR schema's op_attention and slot_kv carry
  it beside `window`): with a window, the first `sinks` keys stay visible, as
  StreamingLLM keeps its initial tokens. 0 or absent means none.
* position_bias and relative_kv (not catalogue params: the IR schema's
  attention op lists them without a rule) are read as T5's bucketed relative
  position bias and Shaw et al.'s relative key/value embeddings; see the
  core's header comment for the exact terms.
* ALiBi: alibiSlopes wins over alibiMax, which wins over alibi. The slopes
  enter as f32 values, as every tensor and number of the op is f32
  (catalogue convention: tensors are row-major f32); the same holds for
  scale and softcap.

Readings where the pages are silent are listed in the module docstrings of
`oracle.alibi` and in the core's header comment. Parity unpinned: a row with
no visible key gives 0, a reading that no page fact and no published method
can confirm. (Non-causal ALiBi uses -slope * |pos - s|, MPT's bidirectional
form; the tests pin it against MPT's own construction of that bias.)
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

from . import alibi as _alibi

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


class _Args(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("S", ctypes.c_int64), ("H", ctypes.c_int64),
        ("G", ctypes.c_int64), ("D", ctypes.c_int64), ("Dv", ctypes.c_int64),
        ("causal", ctypes.c_int32), ("pos_offset", ctypes.c_int64),
        ("scale", ctypes.c_double), ("softcap", ctypes.c_double),
        ("window", ctypes.c_int64), ("slopes", ctypes.POINTER(ctypes.c_double)),
        ("bias_kind", ctypes.c_int32), ("sinks", ctypes.c_int64),
        ("pb_weight", ctypes.c_void_p), ("pb_bounds", ctypes.c_void_p), ("pb_n", ctypes.c_int64),
        ("pb_bidirectional", ctypes.c_int32),
        ("rel_k", ctypes.c_void_p), ("rel_v", ctypes.c_void_p), ("rel_max", ctypes.c_int64),
    ]


def build() -> str:
    """Compile the oracle core with gcc (plain -O2, no fast-math). Each process
    writes its own temporary file and renames it into place, so test workers
    that rebuild at the same time never load a half-written library."""
    tmp = f"{_LIB}.tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [
            ctypes.POINTER(_Args), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def f32(x: float) -> float:
    """The f32 value nearest to x, as a Python float."""
    return float(np.float32(x))


def resolve(T: int, S: int, *, heads: int, headDim: int, kvHeads: Optional[int] = None,
            vHeadDim: Optional[int] = None, causal: Optional[bool] = None,
            posOffset: Optional[int] = None, scale: Optional[float] = None,
            softcap: Optional[float] = None, window: Optional[int] = None,
            alibi: Optional[bool] = None, alibiMax: Optional[float] = None,
            alibiSlopes: Optional[Sequence[float]] = None, sinks: Optional[int] = None) -> dict:
    """Apply the catalogue's defaults; raise ValueError on what it cannot mean."""
    H = int(heads)
    G = int(kvHeads) if kvHeads else H
    D = int(headDim)
    Dv = int(vHeadDim) if vHeadDim else D
    if H <= 0 or G <= 0 or D <= 0 or Dv <= 0 or T < 0 or S < 0:
        raise ValueError("heads, kvHeads, headDim and vHeadDim must be positive")
    if H % G:
        raise ValueError("heads must be a multiple of kvHeads")
    P0 = int(posOffset) if posOffset is not None else 0
    if P0 < 0:
        raise ValueError("posOffset must be >= 0")
    c = float(softcap) if softcap else 0.0
    if c < 0:
        raise ValueError("softcap must be >= 0")
    w = int(window) if window else 0
    if w < 0:
        raise ValueError("window must be >= 0")
    nsink = int(sinks) if sinks else 0
    if nsink < 0:
        raise ValueError("sinks must be >= 0")
    sigma = f32(scale) if scale is not None else f32(1.0 / math.sqrt(D))
    if alibiSlopes is not None:
        if len(alibiSlopes) != H:
            raise ValueError("alibiSlopes must hold one slope per head")
        slopes = [f32(m) for m in alibiSlopes]
    elif alibiMax is not None:
        slopes = [f32(m) for m in _alibi.mpt_slopes(H, float(alibiMax))]
    elif alibi:
        slopes = [f32(m) for m in _alibi.bloom_slopes(H)]
    else:
        slopes = None
    return dict(T=int(T), S=int(S), H=H, G=G, D=D, Dv=Dv,
                causal=True if causal is None else bool(causal), P0=P0,
                scale=sigma, softcap=f32(c), window=w, slopes=slopes, sinks=nsink)


def _position_bias(pb: dict, H: int):
    """(weight f32 [rows, H], thresholds int64, n, bidirectional) of a position_bias
    {weight, buckets, bidirectional?}; buckets are ascending distance thresholds from 0."""
    bounds = np.ascontiguousarray(pb["buckets"], dtype=np.int64)
    n = bounds.size
    if n < 1 or bounds[0] != 0 or np.any(np.diff(bounds) <= 0):
        raise ValueError("position_bias.buckets must be ascending distance thresholds starting at 0")
    bidir = bool(pb.get("bidirectional", False))
    weight = np.ascontiguousarray(pb["weight"], dtype=np.float32)
    if weight.shape != ((2 * n if bidir else n), H):
        raise ValueError(f"position_bias.weight {weight.shape} is not [{2 * n if bidir else n}, heads]")
    return weight, bounds, n, bidir


def _relative_kv(rk: dict, D: int, Dv: int):
    """(key f32 [2m+1, D], value f32 [2m+1, Dv] or None, m) of a relative_kv
    {key, value?, max_distance}."""
    m = int(rk["max_distance"])
    if m < 0:
        raise ValueError("relative_kv.max_distance must be >= 0")
    key = np.ascontiguousarray(rk["key"], dtype=np.float32)
    if key.shape != (2 * m + 1, D):
        raise ValueError(f"relative_kv.key {key.shape} is not [2*max_distance+1, headDim]")
    val = rk.get("value")
    if val is not None:
        val = np.ascontiguousarray(val, dtype=np.float32)
        if val.shape != (2 * m + 1, Dv):
            raise ValueError(f"relative_kv.value {val.shape} is not [2*max_distance+1, vHeadDim]")
    return key, val, m


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, bias: Optional[np.ndarray] = None,
              *, rows: Optional[Sequence[int]] = None, threads: Optional[int] = None,
              position_bias: Optional[dict] = None, relative_kv: Optional[dict] = None,
              **params) -> np.ndarray:
    """The op's output in f64: [T, heads*vHeadDim], or [len(rows), ...] for a row subset.

    q [T, heads*headDim], k [S, kvHeads*headDim], v [S, kvHeads*vHeadDim] and the
    optional bias [T, S] or [heads, T, S] are f32 arrays (catalogue: `attention`
    inputs). `rows` selects query rows to compute (each keeps its own position).
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    T, S = q.shape[0], k.shape[0]
    r = resolve(T, S, **params)
    H, G, D, Dv = r["H"], r["G"], r["D"], r["Dv"]
    if q.shape != (T, H * D) or k.shape != (S, G * D) or v.shape != (S, G * Dv):
        raise ValueError(f"shapes q{q.shape} k{k.shape} v{v.shape} do not match the params")
    bias_kind = 0
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape == (T, S):
            bias_kind = 1
        elif bias.shape == (H, T, S):
            bias_kind = 2
        else:
            raise ValueError(f"bias shape {bias.shape} is neither [T,S] nor [heads,T,S]")
    if rows is None:
        rows_arr = None
        nrows = T
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        if rows_arr.size and (rows_arr.min() < 0 or rows_arr.max() >= T):
            raise ValueError("row index out of range")
        nrows = rows_arr.size
    out = np.zeros((nrows, H * Dv), dtype=np.float64)
    if nrows == 0:
        return out

    slopes_arr = None
    args = _Args(T=T, S=S, H=H, G=G, D=D, Dv=Dv, causal=int(r["causal"]),
                 pos_offset=r["P0"], scale=r["scale"], softcap=r["softcap"],
                 window=r["window"], slopes=None, bias_kind=bias_kind, sinks=r["sinks"])
    if r["slopes"] is not None:
        slopes_arr = np.asarray(r["slopes"], dtype=np.float64)
        args.slopes = slopes_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    keep = []
    if position_bias is not None:
        weight, bounds, n, bidir = _position_bias(position_bias, H)
        keep += [weight, bounds]
        args.pb_weight, args.pb_bounds, args.pb_n = weight.ctypes.data, bounds.ctypes.data, n
        args.pb_bidirectional = int(bidir)
    if relative_kv is not None:
        key, val, m = _relative_kv(relative_kv, D, Dv)
        keep += [key, val]
        args.rel_k, args.rel_max = key.ctypes.data, m
        args.rel_v = val.ctypes.data if val is not None else None

    lib = _load()
    rc = lib.oracle_attention(
        ctypes.byref(args), q.ctypes.data, k.ctypes.data if S else None,
        v.ctypes.data if S else None, bias.ctypes.data if bias is not None else None,
        rows_arr.ctypes.data if rows_arr is not None else None, nrows, out.ctypes.data,
        int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_attention failed with code {rc}")
    return out


def cache_write(cache: np.ndarray, values: np.ndarray, offset: int) -> np.ndarray:
    """Catalogue op `cache_write`: rows [offset, offset+rows) of the cache become
    `values`, in place, and the cache is returned. An exact copy."""
    rows = values.shape[0]
    if values.ndim != 2 or cache.ndim != 2 or values.shape[1] != cache.shape[1]:
        raise ValueError("cache and values must be [*, width] with the same width")
    if offset < 0 or offset + rows > cache.shape[0]:
        raise ValueError("rows past the end of the cache")
    cache[offset:offset + rows] = values
    return cache


from .rope import rope, table as rope_table  # noqa: E402  (op `rope`)
