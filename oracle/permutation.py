"""Seeded uniform permutation sigma (oracle side).  TEST INFRASTRUCTURE ONLY.

[SA-ja] 中核メカニズム step 1 (Permute): for every layer, independently, draw
sigma ~ Uniform(S_n) and reorder the Q, K, V token rows by it.  The page names no generator;
both the oracle and the product implement the same published one, each from its definition:

* splitmix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014; the 64-bit finaliser as published by Vigna): the state advances by the
  golden-ratio increment 0x9E3779B97F4A7C15 and each output is the state passed through a
  xor-shift/multiply finaliser.  Arithmetic is modulo 2^64; the initial state is the seed.
* Fisher-Yates in Durstenfeld's in-place form: walk i from n-1 down to 1 and swap entry i
  with a uniformly chosen entry j in [0, i].  j is drawn by Lemire's multiply-high map
  j = floor(r * (i + 1) / 2^64) of a 64-bit output r (no rejection step; the bias is at most
  n / 2^64, far below anything measurable).

Convention (gather): sigma[p] is the ORIGINAL index of the token placed at permuted slot p,
so the permuted sequence is X_pi[p] = X[sigma[p]] and un-permuting writes Y[sigma[p]] =
Y_pi[p].  This is the reading of "reorder by sigma" / "apply sigma^-1 to the output".

Plain Python integers throughout, so the modulo-2^64 arithmetic is exact and easy to check.
"""

from __future__ import annotations

import numpy as np

_MASK64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB


def splitmix64_stream(seed: int, count: int) -> list[int]:
    """First ``count`` outputs of splitmix64 started from state ``seed``."""
    state = seed & _MASK64
    out = []
    for _ in range(count):
        state = (state + _GOLDEN_GAMMA) & _MASK64
        z = state
        z = ((z ^ (z >> 30)) * _MIX1) & _MASK64
        z = ((z ^ (z >> 27)) * _MIX2) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def fisher_yates(seed: int, n: int) -> list[int]:
    """Durstenfeld shuffle of [0, n) driven by splitmix64(seed); returns the shuffled list."""
    if n < 0:
        raise ValueError("n must be >= 0")
    a = list(range(n))
    if n < 2:
        return a
    draws = splitmix64_stream(seed, n - 1)
    for step, i in enumerate(range(n - 1, 0, -1)):
        j = (draws[step] * (i + 1)) >> 64
        a[i], a[j] = a[j], a[i]
    return a


def make_permutation(seed: int, n: int) -> np.ndarray:
    """sigma as int32[n]: sigma[p] = original token index at permuted slot p."""
    return np.asarray(fisher_yates(seed, n), dtype=np.int32)


def inverse_permutation(sigma: np.ndarray) -> np.ndarray:
    """sigma^-1 as int32[n]: inv[sigma[p]] = p ([SA-ja] 中核メカニズム step 3, Undo Permute)."""
    sigma = np.asarray(sigma)
    n = sigma.shape[0]
    inv = np.full(n, -1, dtype=np.int64)
    for p in range(n):
        inv[int(sigma[p])] = p
    if (inv < 0).any():
        raise ValueError("sigma is not a permutation of [0, n)")
    return inv.astype(np.int32)
