"""One decode step of SA / SWA / the gated layer over a KV cache, float64 (oracle).
TEST INFRASTRUCTURE ONLY.

The pages apply SA to pretrained Qwen3 models without training, which means generating tokens
one at a time from a cache ([SA-ja] 主要な貢献 item 3 and 結果, Qwen3 における推論).  They do not
say how sigma behaves as the cache grows.

Reading (R20): sigma is drawn once per layer over the full context length n_max.  The token at
position t is decoded as row t of causal SA over that length.  Its neighbours are the tokens at
slots within w - 1 of sigma^-1(t) whose original position is <= t ([SA-ja] 中核メカニズム steps
1-3 and 理論的性質 › 因果的制約).  Every such token precedes t, so it is already in the cache, and
decoding t gives exactly the row that a causal forward pass over the whole sequence would give
it.  SWA decoding attends to the w positions [t - w + 1, t] ([HYB]).

Layouts: q [B, Hq, d] (the new token of each batch row), k_cache and v_cache [B, n_max, Hkv, d]
(positions 0..t filled), pos int[B] (t of each row), gates [2, B, Hq].  Output [B, Hq, d].

Pins (tests/test_oracle_decode.py): the decode row equals row t of the pinned forward on the
same tokens; the SWA step and full-window SA step equal torch SDPA over the cache prefix; the
identity sigma reduces SA to SWA; the step never reads past t.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _attend_row, _exact, _f64, sa_neighbours, swa_neighbours
from .permutation import inverse_permutation


def _check(q, k_cache, v_cache, pos):
    if q.ndim != 3 or k_cache.ndim != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q [B, Hq, d], caches [B, n_max, Hkv, d]")
    b_, hq, d = q.shape
    if k_cache.shape[0] != b_ or k_cache.shape[3] != d or hq % k_cache.shape[2] != 0:
        raise ValueError("cache shape does not match q")
    pos = np.asarray(pos, dtype=np.int64)
    n_max = k_cache.shape[1]
    if pos.shape != (b_,) or (pos < 0).any() or (pos >= n_max).any():
        raise ValueError("pos must hold one position in [0, n_max) per batch row")
    return b_, hq, d, n_max, pos


def sa_decode(q, k_cache, v_cache, sigma, window: int, pos, gate=None) -> np.ndarray:
    """Y[b] = attention of q[b] over N~^sigma_w(pos[b]) in the cache of batch row b (R20).

    gate [B, Hq] (optional) multiplies each head's output.
    """
    q, k_cache, v_cache = _exact(q), _exact(k_cache), _exact(v_cache)
    b_, hq, d, n_max, pos = _check(q, k_cache, v_cache, pos)
    sigma = np.asarray(sigma)
    if sigma.shape != (n_max,):
        raise ValueError("sigma must have n_max entries")
    inv = inverse_permutation(sigma)
    out = np.empty((b_, hq, d))
    for b in range(b_):
        idx = sa_neighbours(sigma, window, True, int(pos[b]), inv)
        out[b] = _attend_row(q[b], k_cache[b], v_cache[b], idx, 1.0 / math.sqrt(d))
    if gate is not None:
        out = out * _f64(gate)[..., None]
    return out


def swa_decode(q, k_cache, v_cache, window: int, pos, gate=None) -> np.ndarray:
    """Y[b] = attention of q[b] over cache positions [pos[b] - w + 1, pos[b]] ([HYB])."""
    q, k_cache, v_cache = _exact(q), _exact(k_cache), _exact(v_cache)
    b_, hq, d, n_max, pos = _check(q, k_cache, v_cache, pos)
    out = np.empty((b_, hq, d))
    for b in range(b_):
        idx = swa_neighbours(n_max, window, True, int(pos[b]))
        out[b] = _attend_row(q[b], k_cache[b], v_cache[b], idx, 1.0 / math.sqrt(d))
    if gate is not None:
        out = out * _f64(gate)[..., None]
    return out


def gated_decode(q, k_cache, v_cache, sigma, window: int, pos, gates) -> np.ndarray:
    """Y = g_sa * SA step + g_swa * SWA step, gates [2, B, Hq] ([SA-ja] ゲート付き SA と SWA)."""
    gates = _f64(gates)
    return (sa_decode(q, k_cache, v_cache, sigma, window, pos, gates[0]) +
            swa_decode(q, k_cache, v_cache, window, pos, gates[1]))
