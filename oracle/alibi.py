"""ALiBi slope tables for the oracle (test infrastructure only).

The op catalogue's `attention` entry offers three ways to ask for ALiBi
(param `alibi`: BLOOM's slopes; param `alibiMax`: MPT's slopes from an
alibi_bias_max, typically 8; param `alibiSlopes`: one slope per head given
outright) but defines none of them. The published definitions are used:

* BLOOM / the ALiBi paper (Press, Smith and Lewis, "Train Short, Test Long"):
  with p the largest power of two not above H, head i (1-based) of the first
  p gets 2^(-8 i / p); when H > p the remaining H - p heads take every other
  term, 2^(-4 j / p) for j = 1, 3, 5, ..., of the sequence for 2p heads.
* MPT (`alibi_bias_max` b): with n the smallest power of two not below H,
  head i of n gets 2^(-i b / n); when n != H the even-numbered slopes come
  first, then the odd-numbered ones, and the first H are kept.

Reading taken: the bias a slope produces is -slope * |pos - s| (see the
oracle core). On causal rows this differs from BLOOM's +slope*s and MPT's
slope*(s - (S-1)) forms only by a per-row constant, which the softmax
removes.
"""

from __future__ import annotations

from typing import List


def _floor_pow2(n: int) -> int:
    return 1 << (n.bit_length() - 1)


def _ceil_pow2(n: int) -> int:
    return 1 << (n - 1).bit_length()


def bloom_slopes(heads: int) -> List[float]:
    if heads <= 0:
        raise ValueError("heads must be positive")
    p = _floor_pow2(heads)
    slopes = [2.0 ** (-8.0 * i / p) for i in range(1, p + 1)]
    odd = 1
    while len(slopes) < heads:
        slopes.append(2.0 ** (-4.0 * odd / p))
        odd += 2
    return slopes


def mpt_slopes(heads: int, bias_max: float = 8.0) -> List[float]:
    if heads <= 0:
        raise ValueError("heads must be positive")
    n = _ceil_pow2(heads)
    table = [2.0 ** (-i * bias_max / n) for i in range(1, n + 1)]
    if n != heads:
        evens = [table[i - 1] for i in range(2, n + 1, 2)]
        odds = [table[i - 1] for i in range(1, n + 1, 2)]
        table = (evens + odds)[:heads]
    return table
