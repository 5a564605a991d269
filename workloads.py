"""Seeded synthetic inputs for the attention op and its KV-cache companion.

This module only draws numbers and names shapes. It holds none of the
attention arithmetic, so both sides of a parity check (the CPU oracle and
the HIP library) can take their inputs from here without sharing any of
the method.

Recipe: every tensor is drawn from its own stream,
``numpy.random.default_rng(SeedSequence([seed, tensor_id]))``, as float32
standard normal values times a standard deviation. Stream ids: q = 0, k = 1,
v = 2, bias = 3, bias mask = 4. A bias mask sets an entry to -1e9 with the
stated probability, which is how the op catalogue says to mask a score with
its bias input (graph protocol op catalogue, `attention` inputs).

The pages name no dataset; these Gaussian tensors stand in for activations.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_BIAS, STREAM_BIAS_MASK = 0, 1, 2, 3, 4
STREAM_K_B, STREAM_V_B = 5, 6  # latent attention's per-head up-projections
MASK_VALUE = -1e9


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(stream)]))


def normal(shape, seed: int, stream: int, std: float = 1.0) -> np.ndarray:
    """float32 i.i.d. N(0, std^2) of the given shape."""
    x = rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return np.ascontiguousarray(x, dtype=np.float32)


def masked_bias(shape, seed: int, mask_prob: float, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) bias with each entry set to -1e9 with probability mask_prob."""
    b = normal(shape, seed, STREAM_BIAS, std)
    if mask_prob > 0.0:
        drop = rng(seed, STREAM_BIAS_MASK).random(size=shape) < mask_prob
        b[drop] = np.float32(MASK_VALUE)
    return b


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention call: shapes, op parameters and the input recipe.

    Parameter names follow the op catalogue's `attention` entry (heads,
    headDim, kvHeads, vHeadDim, causal, posOffset, scale, softcap, window,
    alibi, alibiMax, alibiSlopes) plus the input tensor shapes.
    """

    name: str
    T: int
    S: int
    heads: int
    headDim: int
    kvHeads: Optional[int] = None
    vHeadDim: Optional[int] = None
    causal: bool = True
    posOffset: int = 0
    scale: Optional[float] = None
    softcap: Optional[float] = None
    window: Optional[int] = None
    sinks: Optional[int] = None
    alibi: Optional[bool] = None
    alibiMax: Optional[float] = None
    alibiSlopes: Optional[tuple] = None
    bias: Optional[str] = None  # None, "TS" ([T,S]) or "HTS" ([heads,T,S])
    bias_mask_prob: float = 0.0
    std: float = 1.0
    cache_rows: Optional[int] = None  # KV rows in the cache (S) that hold data; None = all
    seed: int = 0

    @property
    def G(self) -> int:
        return self.kvHeads if self.kvHeads else self.heads

    @property
    def Dv(self) -> int:
        return self.vHeadDim if self.vHeadDim else self.headDim

    def params(self) -> dict:
        """The op parameters as keyword arguments (absent ones omitted)."""
        out = {"heads": self.heads, "headDim": self.headDim}
        for key in ("kvHeads", "vHeadDim", "posOffset", "scale", "softcap",
                    "window", "sinks", "alibi", "alibiMax", "alibiSlopes"):
            val = getattr(self, key)
            if val is not None:
                out[key] = val
        out["causal"] = self.causal
        return out

    def tensors(self):
        """(q, k, v, bias or None) as float32 host arrays."""
        H, G, D, Dv = self.heads, self.G, self.headDim, self.Dv
        q = normal((self.T, H * D), self.seed, STREAM_Q, self.std)
        k = normal((self.S, G * D), self.seed, STREAM_K, self.std)
        v = normal((self.S, G * Dv), self.seed, STREAM_V, self.std)
        if self.bias is None:
            bias = None
        elif self.bias == "TS":
            bias = masked_bias((self.T, self.S), self.seed, self.bias_mask_prob)
        elif self.bias == "HTS":
            bias = masked_bias((H, self.T, self.S), self.seed, self.bias_mask_prob)
        else:
            raise ValueError(f"unknown bias layout {self.bias!r}")
        return q, k, v, bias

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class MlaWorkload:
    """One latent (MLA) attention call: the IR schema's op_mla_attention
    properties (heads, kv_rank, qk_nope, qk_rope, v_head_dim, scale, causal,
    window, sinks) plus posOffset and the tensor shapes.

    Recipe: q [T, heads*(qk_nope+qk_rope)] (stream 0) and the latent state
    [S, kv_rank+qk_rope] (stream 1) are N(0, 1); the up-projections k_b
    [heads, qk_nope, kv_rank] (stream 5) and v_b [heads, v_head_dim, kv_rank]
    (stream 6) are N(0, 1/kv_rank), a random initialisation that keeps the
    materialized keys and values at unit scale.
    """

    name: str
    T: int
    S: int
    heads: int
    kv_rank: int
    qk_nope: int
    qk_rope: int
    v_head_dim: int
    causal: Optional[bool] = None
    posOffset: Optional[int] = None
    scale: Optional[float] = None
    window: Optional[int] = None
    sinks: Optional[int] = None
    seed: int = 0

    def params(self) -> dict:
        out = {"heads": self.heads, "kv_rank": self.kv_rank, "qk_nope": self.qk_nope,
               "qk_rope": self.qk_rope, "v_head_dim": self.v_head_dim}
        for key in ("causal", "posOffset", "scale", "window", "sinks"):
            val = getattr(self, key)
            if val is not None:
                out[key] = val
        return out

    def tensors(self):
        """(q, state, k_b, v_b) as float32 host arrays."""
        H, R, N, P, Dv = self.heads, self.kv_rank, self.qk_nope, self.qk_rope, self.v_head_dim
        wstd = 1.0 / float(np.sqrt(R))
        q = normal((self.T, H * (N + P)), self.seed, STREAM_Q)
        state = normal((self.S, R + P), self.seed, STREAM_K)
        k_b = normal((H, N, R), self.seed, STREAM_K_B, wstd)
        v_b = normal((H, Dv, R), self.seed, STREAM_V_B, wstd)
        return q, state, k_b, v_b

    def replace(self, **kw) -> "MlaWorkload":
        return dataclasses.replace(self, **kw)


# The workloads the measurements and the full-size parity tests use.
TINY = Workload("tiny causal prefill T=S=8 H=4 G=2 D=16",
                T=8, S=8, heads=4, kvHeads=2, headDim=16)

LLAMA_DECODE = Workload("llama3-8b-shaped GQA decode T=1 S=32768 H=32 G=8 D=128",
                        T=1, S=32768, heads=32, kvHeads=8, headDim=128,
                        posOffset=32767)

LLAMA_STREAMING = Workload("llama3-8b-shaped streaming decode: window 4096 + 4 sinks over S=32768",
                           T=1, S=32768, heads=32, kvHeads=8, headDim=128, posOffset=32767,
                           window=4096, sinks=4)

# Wide grouped-query groups: 8 query heads per KV head (Llama-3-70B's 64/8)
# and 7 (Qwen2-7B's 28/4), each KV row read once for the whole group.
LLAMA70_DECODE = Workload("llama3-70b-shaped GQA decode T=1 S=32768 H=64 G=8 D=128",
                          T=1, S=32768, heads=64, kvHeads=8, headDim=128, posOffset=32767)

QWEN2_DECODE = Workload("qwen2-7b-shaped GQA decode T=1 S=32768 H=28 G=4 D=128",
                        T=1, S=32768, heads=28, kvHeads=4, headDim=128, posOffset=32767)

LLAMA_PREFILL = Workload("llama3-8b-shaped causal prefill T=S=4096 H=32 G=8 D=128",
                         T=4096, S=4096, heads=32, kvHeads=8, headDim=128)

LLAMA_CHUNKED = Workload("llama3-8b-shaped chunked prefill T=512 at 3584, S=4096",
                         T=512, S=4096, heads=32, kvHeads=8, headDim=128,
                         posOffset=3584)

GEMMA2_SWA = Workload("gemma2-shaped sliding-window prefill T=S=8192 H=16 G=8 D=256",
                      T=8192, S=8192, heads=16, kvHeads=8, headDim=256,
                      scale=256 ** -0.5, softcap=50.0, window=4096, std=2.0)

LATENT_DECODE = Workload("latent-shaped ALiBi+bias decode T=1 S=8192 H=16 D=192 Dv=128",
                         T=1, S=8192, heads=16, kvHeads=16, headDim=192,
                         vHeadDim=128, posOffset=8191, alibi=True, bias="HTS",
                         bias_mask_prob=0.1)

LATENT_NONCAUSAL = Workload("latent-shaped ALiBi+bias non-causal T=S=1024 H=16 D=192 Dv=128",
                            T=1024, S=1024, heads=16, kvHeads=16, headDim=192,
                            vHeadDim=128, causal=False, alibi=True, bias="HTS",
                            bias_mask_prob=0.1)

ALL = (TINY, LLAMA_DECODE, LLAMA_PREFILL, LLAMA_CHUNKED, GEMMA2_SWA,
       LATENT_DECODE, LATENT_NONCAUSAL)

# Latent attention in absorbed form over the same model shape as the
# latent-shaped decode above (DeepSeek-V2-Lite: 16 heads, kv_rank 512,
# qk_nope 128, qk_rope 64, v_head_dim 128): a 576-float latent row per key
# instead of 16 heads x (192 + 128) floats.
MLA_DECODE = MlaWorkload("deepseek-v2-lite-shaped absorbed MLA decode T=1 S=8192 H=16 kv_rank=512",
                         T=1, S=8192, heads=16, kv_rank=512, qk_nope=128, qk_rope=64,
                         v_head_dim=128, posOffset=8191)

# The same at DeepSeek-V3's 128 heads over a 32768-row latent cache: eight
# 16-head blocks share every latent row, so the matrix cores bound it.
MLA_DECODE_V3 = MlaWorkload("deepseek-v3-shaped absorbed MLA decode T=1 S=32768 H=128 kv_rank=512",
                            T=1, S=32768, heads=128, kv_rank=512, qk_nope=128, qk_rope=64,
                            v_head_dim=128, posOffset=32767)
