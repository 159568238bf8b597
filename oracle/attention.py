"""Stochastic Attention / SWA / gated SA+SWA forward in float64 (oracle).  TEST INFRASTRUCTURE ONLY.

Written from the pages' definitions, one query row at a time, with no blocking, fusion or
reordering.  Notation follows the pages: sigma is the per-layer permutation, w the window,
N~^sigma_w(i) the random neighbourhood of original position i.

Layouts (token-major, "BSHD"): q [B, n, Hq, d]; k, v [B, n, Hkv, d]; sigma int[n];
gates [2, B, n, Hq] with g_sa first.  Outputs are float64 [B, n, Hq, d].

Readings of points the pages leave open (each one is also listed in the design notes):
  R1 gather convention: X_pi[p] = X[sigma[p]], Y[sigma[p]] = Y_pi[p].
  R2 the window in permuted space is the band |p - q| <= w - 1 (both modes); in causal mode a
     key is kept only if it also precedes the query in ORIGINAL order.  With sigma = identity
     this is exactly the causal SWA of [HYB] (the w tokens up to and including t).
  R3 the causal test is sigma[q] <= sigma[p] ("<=" keeps the token itself).
  R4 the band is truncated at both sequence ends (no wrap-around).
  R5 softmax scale 1/sqrt(d), no soft-capping.
  R7 GQA: query head h reads KV head floor(h / G), G = Hq / Hkv.
  R8 gates are given values in (0, 1) per (batch, original token, query head), broadcast over d.
  R9 the SWA path of the gated layer uses the same w and causal flag as the SA path.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from .permutation import inverse_permutation


def _f64(x) -> np.ndarray:
    """Exact float64 copy of a NumPy array or a (CPU or device) torch tensor of any float dtype."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _exact(x) -> np.ndarray:
    """A NumPy view holding exactly the values of x, without widening to float64 yet.

    bfloat16 and float32 tensors become float32 arrays (every bfloat16 value is a float32 value),
    float64 stays float64.  Rows are widened to float64 where they enter arithmetic, so large
    inputs need not be copied whole.
    """
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        x = x.numpy() if str(x.dtype) in ("torch.float32", "torch.float64") else x.float().numpy()
    x = np.asarray(x)
    if x.dtype not in (np.float32, np.float64):
        x = x.astype(np.float64)
    return x


# ----------------------------------------------------------------------------------------------
# Neighbour sets
# ----------------------------------------------------------------------------------------------

def sa_neighbours(sigma: np.ndarray, window: int, causal: bool, i: int,
                  inv: Optional[np.ndarray] = None) -> np.ndarray:
    """Original indices j that original position i attends to under SA: N~^sigma_w(i).

    [SA-ja] 中核メカニズム: after the permutation, standard window attention runs in the
    permuted space, so the query sitting at slot p = sigma^-1(i) sees the keys at the slots of
    its window (R2: |p - q| <= w - 1, truncated at the ends, R4); the token at slot q is the
    original token sigma[q].  [SA-ja] 理論的性質 (因果的制約): in the autoregressive setting only
    causally reachable tokens are kept, i.e. sigma[q] <= i (R3).
    Returned sorted ascending.
    """
    sigma = np.asarray(sigma)
    n = sigma.shape[0]
    if inv is None:
        inv = inverse_permutation(sigma)
    p = int(inv[i])
    lo = max(0, p - (window - 1))
    hi = min(n - 1, p + (window - 1))
    members = sigma[lo:hi + 1].astype(np.int64)
    if causal:
        members = members[members <= i]
    return np.sort(members)


def swa_neighbours(n: int, window: int, causal: bool, i: int) -> np.ndarray:
    """Original indices j that position i attends to under plain sliding-window attention.

    [HYB] ハイブリッドアーキテクチャの定義: the SWA output at position t is restricted to the w
    tokens just before it -- read as j in [t - w + 1, t] (the token itself included, so exactly w
    keys away from the start).  The non-causal form is the two-sided band |i - j| <= w - 1 (R2).
    """
    lo = max(0, i - (window - 1))
    hi = i if causal else min(n - 1, i + (window - 1))
    return np.arange(lo, hi + 1, dtype=np.int64)


# ----------------------------------------------------------------------------------------------
# One output row
# ----------------------------------------------------------------------------------------------

def _attend_row(q_i: np.ndarray, k_b: np.ndarray, v_b: np.ndarray, idx: np.ndarray,
                scale: float) -> np.ndarray:
    """softmax_j(scale * <q_i[h], K[j, kv(h)]>) weighted sum of V[j, kv(h)] over j in idx.

    q_i [Hq, d]; k_b, v_b [n, Hkv, d]; idx int[m].  Returns [Hq, d].  The softmax subtracts
    the row maximum before exponentiating (the value is unchanged by it).
    """
    q_i = q_i.astype(np.float64)
    hq, d = q_i.shape
    hkv = k_b.shape[1]
    g = hq // hkv
    kj = k_b[idx].astype(np.float64)                # [m, Hkv, d]
    vj = v_b[idx].astype(np.float64)                # [m, Hkv, d]
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        kvh = h // g                                # R7
        s = scale * (kj[:, kvh, :] @ q_i[h])        # [m]
        s = s - s.max()
        e = np.exp(s)
        out[h] = (e @ vj[:, kvh, :]) / e.sum()
    return out


def _rows_or_all(n: int, rows: Optional[Iterable[int]]) -> np.ndarray:
    return np.arange(n, dtype=np.int64) if rows is None else np.asarray(list(rows), dtype=np.int64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, n, H, d]")
    b, n, hq, d = q.shape
    if k.shape[:2] != (b, n) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError("k, v must be [B, n, Hkv, d] matching q")
    if hq % k.shape[2] != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return b, n, hq, d


def sa_rows(q, k, v, sigma, window: int, causal: bool,
            rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Y_sa at the given ORIGINAL token indices (all of them if rows is None): [B, len(rows), Hq, d].

    [SA-ja] 中核メカニズム steps 1-3 + 理論的性質 (因果的制約), evaluated in original token space:
    Y_sa[i] = sum over j in N~^sigma_w(i) of softmax_j(<Q_i, K_j>/sqrt(d)) V_j   (R5).
    """
    q, k, v = _exact(q), _exact(k), _exact(v)
    b_, n, hq, d = _check_shapes(q, k, v)
    if window < 1:
        raise ValueError("window must be >= 1")
    sigma = np.asarray(sigma)
    if sigma.shape != (n,):
        raise ValueError("sigma must have n entries")
    inv = inverse_permutation(sigma)
    scale = 1.0 / math.sqrt(d)
    rows = _rows_or_all(n, rows)
    out = np.empty((b_, rows.shape[0], hq, d), dtype=np.float64)
    for r, i in enumerate(rows):
        idx = sa_neighbours(sigma, window, causal, int(i), inv)
        for b in range(b_):
            out[b, r] = _attend_row(q[b, i], k[b], v[b], idx, scale)
    return out


def swa_rows(q, k, v, window: int, causal: bool,
             rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Y_swa at the given original token indices: plain sliding-window attention ([HYB], R2)."""
    q, k, v = _exact(q), _exact(k), _exact(v)
    b_, n, hq, d = _check_shapes(q, k, v)
    if window < 1:
        raise ValueError("window must be >= 1")
    scale = 1.0 / math.sqrt(d)
    rows = _rows_or_all(n, rows)
    out = np.empty((b_, rows.shape[0], hq, d), dtype=np.float64)
    for r, i in enumerate(rows):
        idx = swa_neighbours(n, window, causal, int(i))
        for b in range(b_):
            out[b, r] = _attend_row(q[b, i], k[b], v[b], idx, scale)
    return out


def sa_forward(q, k, v, sigma, window: int, causal: bool) -> np.ndarray:
    """Full SA forward, [B, n, Hq, d] float64."""
    return sa_rows(q, k, v, sigma, window, causal, None)


def swa_forward(q, k, v, window: int, causal: bool) -> np.ndarray:
    """Full SWA forward, [B, n, Hq, d] float64."""
    return swa_rows(q, k, v, window, causal, None)


def gated_forward(q, k, v, sigma, window: int, causal: bool, gates,
                  rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Gated dual path Y = g_sa * Y_sa + g_swa * Y_swa ([SA-ja] ゲート付き SA と SWA の組み合わせ).

    gates [2, B, n, Hq] (g_sa first), broadcast over the head dimension d (R8); both paths use
    the same w and causal flag (R9).  Returns [B, len(rows), Hq, d].
    """
    gates = _f64(gates)
    n = q.shape[1]
    rr = _rows_or_all(n, rows)
    y_sa = sa_rows(q, k, v, sigma, window, causal, rr)
    y_swa = swa_rows(q, k, v, window, causal, rr)
    g_sa = gates[0][:, rr, :, None]
    g_swa = gates[1][:, rr, :, None]
    return g_sa * y_sa + g_swa * y_swa


# ----------------------------------------------------------------------------------------------
# Second formulation, in permuted space (dense, small n only)
# ----------------------------------------------------------------------------------------------

def sa_forward_permuted_dense(q, k, v, sigma, window: int, causal: bool) -> np.ndarray:
    """SA computed the way the page's three steps read, with a dense n x n mask.

    Step 1 ([SA-ja] 中核メカニズム, Permute): Q_pi = Q[sigma], K_pi = K[sigma], V_pi = V[sigma].
    Step 2 (window attention in permuted space): mask M[p, q] = (|p - q| <= w - 1) and, when
    causal, sigma[q] <= sigma[p]; masked softmax of Q_pi K_pi^T / sqrt(d); Y_pi = P V_pi.
    Step 3 (Undo Permute): Y[sigma[p]] = Y_pi[p].
    O(n^2) memory: for cross-checking sa_rows on small n only.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    b_, n, hq, d = _check_shapes(q, k, v)
    hkv = k.shape[2]
    g = hq // hkv
    sigma = np.asarray(sigma).astype(np.int64)
    q_pi, k_pi, v_pi = q[:, sigma], k[:, sigma], v[:, sigma]
    slots = np.arange(n)
    mask = np.abs(slots[:, None] - slots[None, :]) <= (window - 1)
    if causal:
        mask &= sigma[None, :] <= sigma[:, None]
    scale = 1.0 / math.sqrt(d)
    y_pi = np.empty_like(q_pi)
    for b in range(b_):
        for h in range(hq):
            s = scale * (q_pi[b, :, h, :] @ k_pi[b, :, h // g, :].T)    # [n, n]
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=1, keepdims=True)
            y_pi[b, :, h, :] = p @ v_pi[b, :, h // g, :]
    y = np.empty_like(y_pi)
    y[:, sigma] = y_pi
    return y
