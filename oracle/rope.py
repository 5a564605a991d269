"""Rotary position embedding: the oracle's definition (test infrastructure only;
the HIP library never imports it).

Graph protocol op catalogue, op `rope`: x [T, heads*headDim] -> same shape;
params headDim, base (rope_theta, default 10000), offset (absolute position
of the first row), rotaryDim, interleaved, scaling (a model config's
rope_scaling object: linear, llama3, yarn, longrope, dynamic), invFreq
(explicit inverse frequencies, rotaryDim/2 of them) and attentionFactor
(multiplies cos and sin).

The page names the parameters; the arithmetic below is the plainest reading
of them, as each model family the page lists defines it:

R1  Row t sits at position offset + t. Within each head the first rotaryDim
    channels form rotaryDim/2 pairs; pair i turns by the angle
    position * invFreq[i]. Channels from rotaryDim on pass through.
R2  Pairing: half-split pairs channel i with i + rotaryDim/2 (Llama, NeoX,
    Qwen, Mistral); interleaved pairs 2i with 2i + 1 (GPT-J, CodeGen, GLM).
R3  Sense of the turn: (a, b) -> (a cos - b sin, a sin + b cos), the
    RoFormer convention (Su et al., 2021, "RoFormer: Enhanced Transformer
    with Rotary Position Embedding", the 2-D rotation of each pair).
R4  Default table: invFreq[i] = base^(-2i/rotaryDim) (RoFormer's theta_i).
R5  attentionFactor scales cos and sin, so it scales the rotated channels
    only; pass-through channels are never multiplied.
R6  Precision: the table and the factor are f32 numbers (catalogue
    convention: f32 everywhere). Each is computed in f64 and rounded to f32
    once. The angle is then the exact product position * invFreq[i] of that
    f32 value, and the turn is exact; the result is returned in f64 and the
    op's f32 output is its rounding.
R7  Anything that depends on the sequence length (dynamic, longrope) uses
    seq_len = offset + T: one more than the largest position in the call.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _theta(rd: int, base: float) -> np.ndarray:
    """RoFormer's frequencies base^(-2i/rd), i < rd/2, in f64 (R4). Python's
    float power (the C library's pow), one entry at a time."""
    return np.array([float(base) ** (-2.0 * i / rd) for i in range(rd // 2)], dtype=np.float64)


def _linear(theta, s):
    """Position interpolation (Chen et al., 2023, "Extending Context Window of
    Large Language Models via Positional Interpolation"): positions are divided
    by the factor, i.e. every frequency is."""
    return theta / float(s["factor"])


def _llama3(theta, s):
    """Llama 3.1's frequency-dependent scaling: wavelengths shorter than
    original/high_freq_factor keep their frequency, longer than
    original/low_freq_factor are divided by `factor`, and in between the two
    are blended linearly in original/wavelength."""
    factor = float(s["factor"])
    lo_f = float(s.get("low_freq_factor", 1.0))
    hi_f = float(s.get("high_freq_factor", 4.0))
    orig = float(s["original_max_position_embeddings"])
    wavelen = 2.0 * math.pi / theta
    out = np.empty_like(theta)
    for i, (f, wl) in enumerate(zip(theta, wavelen)):
        if wl < orig / hi_f:
            out[i] = f
        elif wl > orig / lo_f:
            out[i] = f / factor
        else:
            smooth = (orig / wl - lo_f) / (hi_f - lo_f)
            out[i] = (1.0 - smooth) * f / factor + smooth * f
    return out


def _yarn_mscale(scale: float, k: float = 1.0) -> float:
    """YaRN's attention temperature: 0.1 k ln(s) + 1 for s > 1."""
    return 0.1 * k * math.log(scale) + 1.0 if scale > 1.0 else 1.0


def _yarn(theta, s, rd, base):
    """YaRN (Peng et al., 2023, "YaRN: Efficient Context Window Extension of
    Large Language Models"), NTK-by-parts: a pair that turns more than
    beta_fast times over the original context keeps its frequency, one that
    turns fewer than beta_slow times is interpolated (divided by the factor),
    and a linear ramp over the pair index blends the two in between. The ramp's
    ends are the pair indices at which the turn counts equal beta_fast and
    beta_slow (rounded outwards unless truncate is false)."""
    factor = float(s["factor"])
    orig = float(s["original_max_position_embeddings"])
    b_fast = float(s.get("beta_fast") or 32.0)
    b_slow = float(s.get("beta_slow") or 1.0)

    def index_for(turns):
        # pair i turns orig / (2 pi base^(2i/rd)) times over the original context
        return rd * math.log(orig / (turns * 2.0 * math.pi)) / (2.0 * math.log(base))

    lo, hi = index_for(b_fast), index_for(b_slow)
    if s.get("truncate", True):
        lo, hi = math.floor(lo), math.ceil(hi)
    lo, hi = max(lo, 0), min(hi, rd - 1)
    if lo == hi:
        hi += 0.001
    i = np.arange(rd // 2, dtype=np.float64)
    ramp = np.clip((i - lo) / (hi - lo), 0.0, 1.0)     # 0: keep, 1: interpolate
    return theta * (1.0 - ramp) + (theta / factor) * ramp


def _yarn_factor(s) -> float:
    factor = float(s["factor"])
    m, m_all = s.get("mscale"), s.get("mscale_all_dim")
    if m and m_all:
        return _yarn_mscale(factor, float(m)) / _yarn_mscale(factor, float(m_all))
    return _yarn_mscale(factor)


def _longrope(theta, s, rd, seq_len):
    """LongRoPE (Ding et al., 2024, "LongRoPE: Extending LLM Context Window
    Beyond 2 Million Tokens"), as Phi-3 configs carry it: per-pair rescale
    factors, the long set once the sequence passes the original context, the
    short set before."""
    orig = int(s["original_max_position_embeddings"])
    ext = s["long_factor"] if seq_len > orig else s["short_factor"]
    ext = np.asarray(ext, dtype=np.float64)
    if ext.shape != (rd // 2,):
        raise ValueError("longrope factors must hold rotaryDim/2 values")
    return theta / ext


def _longrope_factor(s) -> float:
    orig = float(s["original_max_position_embeddings"])
    factor = s.get("factor")
    if factor is None:
        factor = float(s["max_position_embeddings"]) / orig
    factor = float(factor)
    return math.sqrt(1.0 + math.log(factor) / math.log(orig)) if factor > 1.0 else 1.0


def _dynamic_base(base, s, rd, seq_len):
    """Dynamic NTK-aware scaling: past the original context the base grows to
    base * (factor * seq_len / original - (factor - 1))^(rd / (rd - 2))."""
    orig = float(s.get("original_max_position_embeddings") or s["max_position_embeddings"])
    factor = float(s["factor"])
    if rd <= 2:
        raise ValueError("dynamic scaling needs rotaryDim > 2")
    if seq_len <= orig:
        return base
    return base * (factor * seq_len / orig - (factor - 1.0)) ** (rd / (rd - 2.0))


def table(rotaryDim: int, *, base: Optional[float] = None, scaling: Optional[dict] = None,
          invFreq: Optional[Sequence[float]] = None, attentionFactor: Optional[float] = None,
          seq_len: int = 1):
    """(invFreq f32 [rotaryDim/2], attention factor as the f64 value of an f32).

    Precedence: an explicit invFreq replaces base and scaling; an explicit
    attentionFactor replaces the scaling's own attention_factor, which replaces
    the one yarn and longrope derive; otherwise 1 (R4-R7)."""
    rd = int(rotaryDim)
    if rd <= 0 or rd % 2:
        raise ValueError("rotaryDim must be positive and even")
    b = 10000.0 if base is None else float(base)
    if b <= 0:
        raise ValueError("base must be > 0")
    af = 1.0
    kind = None
    if scaling:
        kind = scaling.get("rope_type", scaling.get("type"))
    if invFreq is not None:
        inv = np.asarray(invFreq, dtype=np.float64)
        if inv.shape != (rd // 2,):
            raise ValueError("invFreq must hold rotaryDim/2 values")
    elif kind in (None, "default"):
        inv = _theta(rd, b)
    elif kind == "linear":
        inv = _linear(_theta(rd, b), scaling)
    elif kind == "llama3":
        inv = _llama3(_theta(rd, b), scaling)
    elif kind == "yarn":
        inv = _yarn(_theta(rd, b), scaling, rd, b)
        af = _yarn_factor(scaling)
    elif kind == "longrope":
        inv = _longrope(_theta(rd, b), scaling, rd, seq_len)
        af = _longrope_factor(scaling)
    elif kind == "dynamic":
        inv = _theta(rd, _dynamic_base(b, scaling, rd, seq_len))
    else:
        raise ValueError(f"unknown rope scaling {kind!r}")
    if scaling and scaling.get("attention_factor") is not None:
        af = float(scaling["attention_factor"])
    if attentionFactor is not None:
        af = float(attentionFactor)
    return _f32(inv), float(np.float32(af))


def rope(x: np.ndarray, *, headDim: int, base: Optional[float] = None,
         offset: Optional[int] = None, rotaryDim: Optional[int] = None,
         interleaved: Optional[bool] = None, scaling: Optional[dict] = None,
         invFreq: Optional[Sequence[float]] = None,
         attentionFactor: Optional[float] = None) -> np.ndarray:
    """Op `rope` on x [T, heads*headDim] (f32); the result in f64 (R1-R7)."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be [T, heads*headDim]")
    T, W = x.shape
    D = int(headDim)
    if D <= 0 or W % D:
        raise ValueError("the row width must be a multiple of headDim")
    rd = int(rotaryDim) if rotaryDim else D
    if rd > D:
        raise ValueError("rotaryDim must not exceed headDim")
    p0 = int(offset) if offset else 0
    if p0 < 0:
        raise ValueError("offset must be >= 0")
    inv, af = table(rd, base=base, scaling=scaling, invFreq=invFreq,
                    attentionFactor=attentionFactor, seq_len=p0 + T)
    half = rd // 2
    if interleaved:
        ia, ib = 2 * np.arange(half), 2 * np.arange(half) + 1
    else:
        ia, ib = np.arange(half), np.arange(half) + half
    y = x.astype(np.float64).reshape(T, W // D, D)
    out = y.copy()
    pos = (p0 + np.arange(T, dtype=np.int64)).astype(np.float64)
    ang = pos[:, None] * inv.astype(np.float64)[None, :]          # [T, half]
    c = (np.cos(ang) * af)[:, None, :]
    s = (np.sin(ang) * af)[:, None, :]
    a, b = y[:, :, ia], y[:, :, ib]
    out[:, :, ia] = a * c - b * s
    out[:, :, ib] = a * s + b * c
    return out.reshape(T, W)
