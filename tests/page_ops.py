"""The op catalogue's own primitive ops, in numpy f64, for the composition pin.

Each function follows its catalogue entry (graph protocol op catalogue):
`slice` (a contiguous run of the first axis or of the last one), `matmul`
(with `transB`: read b as [out, in]), `scale` (times a constant factor),
`softcap` (cap * tanh(x / cap)), `add` (elementwise; b may be a row vector
or a single value), `causal_mask` (strict upper triangle of each square
block of the last two dims set to -inf) and `softmax` (over the last
dimension, max-subtracted). The attention oracle must equal a composition
of these wherever they can express the op.
"""

import numpy as np


def slice_(a, start, length, axis=0):
    a = np.asarray(a)
    if axis == 0:
        return a[start:start + length]
    if axis in (-1, a.ndim - 1):
        return a[..., start:start + length]
    raise ValueError("slice takes axis 0 or the last axis")


def matmul(a, b, transB=False):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if transB:
        b = b.T
    return a @ b


def scale(a, factor):
    return np.asarray(a, dtype=np.float64) * float(factor)


def softcap(x, cap):
    x = np.asarray(x, dtype=np.float64)
    return cap * np.tanh(x / cap)


def add(a, b):
    return np.asarray(a, dtype=np.float64) + np.asarray(b, dtype=np.float64)


def causal_mask(a):
    a = np.array(a, dtype=np.float64, copy=True)
    n = a.shape[-1]
    if a.shape[-2] != n:
        raise ValueError("causal_mask needs square blocks")
    upper = np.triu(np.ones((n, n), dtype=bool), k=1)
    a[..., upper] = -np.inf
    return a


def softmax(x):
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)
