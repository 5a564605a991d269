"""Latent (MLA) attention oracle, in f64 numpy (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module; the HIP library never does, and the two share no code.

The IR schema page lists an `op_mla_attention` (properties state, heads,
kv_rank, qk_nope, qk_rope, v_head_dim, k_b, v_b, scale, causal, window,
sinks) and the op catalogue's `attention` entry names DeepSeek MLA where it
lets vHeadDim differ from headDim; neither page says what the op computes.
The plainest reading, which this module writes out, is DeepSeek-V2's
multi-head latent attention:

* state [S, kv_rank + qk_rope]: row s is the compressed key/value c_s
  (kv_rank channels) followed by the rotary key part k_pe_s (qk_rope
  channels), which every head shares.
* q [T, heads * (qk_nope + qk_rope)]: head h holds its no-rope part
  (qk_nope channels) then its rotary part (qk_rope channels).
* k_b [heads, qk_nope, kv_rank] and v_b [heads, v_head_dim, kv_rank]: the
  per-head up-projections of c_s into a key and a value.
* Head h attends with key_h(s) = [k_b[h] c_s ; k_pe_s] (qk_nope + qk_rope
  channels) and value_h(s) = v_b[h] c_s (v_head_dim channels), exactly as
  the `attention` op would over those materialized keys and values: score
  scale * q_h . key_h(s) (scale defaults to 1/sqrt(qk_nope + qk_rope), the
  width it replaces), the causal / window / sinks visibility rule, a
  max-subtracted softmax, and out[t, h*v_head_dim + e] the weighted sum; a
  row with no visible key is 0.
* Rotary embeddings of q and k_pe happen before this op (they are already in
  q and state), as the `rope` op does upstream of `attention`.

This is the definition, materialized; the "absorbed" evaluation a fast
kernel uses (q_h's no-rope part multiplied into k_b[h] first, v_b[h] applied
after the softmax) reaches the same result up to rounding, by associativity.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def resolve(T: int, S: int, *, heads: int, kv_rank: int, qk_nope: int, qk_rope: int,
            v_head_dim: int, scale: Optional[float] = None, causal: Optional[bool] = None,
            posOffset: Optional[int] = None, window: Optional[int] = None,
            sinks: Optional[int] = None) -> dict:
    """Defaults and refusals for the op's parameters."""
    H, R, N, P, Dv = int(heads), int(kv_rank), int(qk_nope), int(qk_rope), int(v_head_dim)
    if min(H, R, N, Dv) <= 0 or P < 0 or T < 0 or S < 0:
        raise ValueError("heads, kv_rank, qk_nope and v_head_dim must be positive, qk_rope >= 0")
    P0 = int(posOffset) if posOffset is not None else 0
    if P0 < 0:
        raise ValueError("posOffset must be >= 0")
    w = int(window) if window else 0
    if w < 0:
        raise ValueError("window must be >= 0")
    nsink = int(sinks) if sinks else 0
    if nsink < 0:
        raise ValueError("sinks must be >= 0")
    # The op's numbers are f32 (catalogue convention: tensors are row-major f32).
    sigma = float(np.float32(scale)) if scale is not None else float(np.float32(1.0 / math.sqrt(N + P)))
    return dict(T=int(T), S=int(S), H=H, R=R, N=N, P=P, Dv=Dv,
                causal=True if causal is None else bool(causal), P0=P0, window=w, sinks=nsink,
                scale=sigma)


def visible(causal: bool, window: int, sinks: int, pos: int, S: int) -> np.ndarray:
    """Boolean mask over key rows 0..S-1 for a query at absolute position pos
    (graph protocol op catalogue, op `attention`, params causal and window;
    sinks read as keys s < sinks kept in view beside a window)."""
    s = np.arange(S, dtype=np.int64)
    if window > 0:
        in_window = (s > pos - window) if causal else (np.abs(pos - s) <= window)
        seen = in_window | (s < sinks)
    else:
        seen = np.ones(S, dtype=bool)
    if causal:
        seen &= s <= pos
    return seen


def materialize(state: np.ndarray, k_b: np.ndarray, v_b: np.ndarray, r: dict):
    """Per-head keys [H, S, qk_nope + qk_rope] and values [H, S, v_head_dim], f64."""
    R, N, P, Dv, H = r["R"], r["N"], r["P"], r["Dv"], r["H"]
    c = state[:, :R].astype(np.float64)
    kpe = state[:, R:R + P].astype(np.float64)
    S = state.shape[0]
    keys = np.empty((H, S, N + P))
    vals = np.empty((H, S, Dv))
    for h in range(H):
        keys[h, :, :N] = c @ k_b[h].astype(np.float64).T
        keys[h, :, N:] = kpe
        vals[h] = c @ v_b[h].astype(np.float64).T
    return keys, vals


def mla_attention(q: np.ndarray, state: np.ndarray, k_b: np.ndarray, v_b: np.ndarray, *,
                  rows: Optional[Sequence[int]] = None, **params) -> np.ndarray:
    """The op's output in f64: [T, heads*v_head_dim], or [len(rows), ...]."""
    T, S = q.shape[0], state.shape[0]
    r = resolve(T, S, **params)
    H, R, N, P, Dv = r["H"], r["R"], r["N"], r["P"], r["Dv"]
    if q.shape != (T, H * (N + P)) or state.shape != (S, R + P):
        raise ValueError(f"shapes q{q.shape} state{state.shape} do not match the params")
    if k_b.shape != (H, N, R) or v_b.shape != (H, Dv, R):
        raise ValueError(f"shapes k_b{k_b.shape} v_b{v_b.shape} do not match the params")
    keys, vals = materialize(state, k_b, v_b, r)
    idx = list(range(T)) if rows is None else [int(t) for t in rows]
    out = np.zeros((len(idx), H * Dv))
    for i, t in enumerate(idx):
        if not 0 <= t < T:
            raise ValueError("row index out of range")
        vis = visible(r["causal"], r["window"], r["sinks"], r["P0"] + t, S)
        if not vis.any():
            continue
        for h in range(H):
            qh = q[t, h * (N + P):(h + 1) * (N + P)].astype(np.float64)
            x = r["scale"] * (keys[h][vis] @ qh)
            p = np.exp(x - x.max())
            out[i, h * Dv:(h + 1) * Dv] = (p @ vals[h][vis]) / p.sum()
    return out
