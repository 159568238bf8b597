"""Gradients of SA / SWA / gated SA+SWA in float64 (oracle).  TEST INFRASTRUCTURE ONLY.

The pages pretrain a model from scratch with the gated SA + SWA layer in place ([SA-ja] 主要な
貢献 item 3 and 結果, 事前学習), so the layer needs a backward pass.  No page writes one out.
The layer is an exact function of its inputs for a fixed sigma, so its gradient is fixed by the
forward definition alone:

* the forward is the one in attention.py ([SA-ja] 中核メカニズム steps 1-3, 理論的性質, and the
  gated equation of ゲート付き SA と SWA の組み合わせ);
* the backward below is the chain rule through that definition, one query row at a time.

There is no blocking, fusion or reordering.  For query i, head h, with N = N~^sigma_w(i),
s = 1/sqrt(d), and kv = the KV head of h (R7):

    S_j   = s <Q_i, K_j>                   (j in N)
    P_j   = exp(S_j) / sum_k exp(S_k)
    A_i   = sum_j P_j V_j                  (the attention output of the row)
    y_i   = g_i A_i                        (g = the gate, or 1)

Given dy_i = dL/dy_i:

    dA_i  = g_i dy_i
    dg_i  = <dy_i, A_i>
    dV_j += P_j dA_i
    dP_j  = <dA_i, V_j>
    dS_j  = P_j (dP_j - sum_k P_k dP_k)    (softmax Jacobian; sum_k P_k dP_k = <dA_i, A_i>)
    dQ_i += s sum_j dS_j K_j
    dK_j += s dS_j Q_i

The gated layer is y = g_sa A_sa + g_swa A_swa. Its gradient is the sum of the two paths'
gradients, each taken with its own gate.

The log-sum-exp of a row, lse_i = log sum_j exp(S_j), is what a forward pass hands to a backward
pass so that P can be rebuilt without a second softmax.  It is defined here too.

Layouts are those of attention.py: q, dy [B, n, Hq, d]; k, v [B, n, Hkv, d]; gates [2, B, n, Hq].

Pins (tests/test_oracle_backward.py), none of which reuses the code below:
  * central finite differences of the pinned forward;
  * torch.autograd through torch's scaled_dot_product_attention, with the dense mask built from
    the neighbour sets;
  * closed forms: sum_j dV_j = sum_i g_i dy_i, because every softmax row sums to 1; sum_j dK_j =
    0, because shifting every key by one vector leaves each row unchanged;
    sum <dQ, Q> = sum <dK, K>, because the scores are bilinear in Q and K; dQ = 0 when all V rows
    are equal;
  * planted mistakes, each caught by one of the above.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Tuple

import numpy as np

from .attention import _check_shapes, _exact, _f64, _rows_or_all, sa_neighbours, swa_neighbours
from .permutation import inverse_permutation


def _neighbour_fn(sigma, n: int, window: int, causal: bool):
    """i -> its neighbour set: SA when sigma is given, plain SWA when sigma is None."""
    if sigma is None:
        return lambda i: swa_neighbours(n, window, causal, i)
    sigma = np.asarray(sigma)
    if sigma.shape != (n,):
        raise ValueError("sigma must have n entries")
    inv = inverse_permutation(sigma)
    return lambda i: sa_neighbours(sigma, window, causal, i, inv)


def _row_probs(q_ih: np.ndarray, k_rows: np.ndarray, scale: float) -> Tuple[np.ndarray, float]:
    """P over the row's keys and the row's log-sum-exp.  q_ih [d]; k_rows [m, d]."""
    s = scale * (k_rows @ q_ih)
    mx = s.max()
    e = np.exp(s - mx)
    tot = e.sum()
    return e / tot, mx + math.log(tot)


# ----------------------------------------------------------------------------------------------
# Log-sum-exp of the rows
# ----------------------------------------------------------------------------------------------

def attention_lse_rows(q, k, sigma, window: int, causal: bool,
                       rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """lse[b, r, h] = log sum_{j in N(i)} exp(<Q[b,i,h], K[b,j,kv(h)]> / sqrt(d)), i = rows[r].

    SA when sigma is given, plain SWA when sigma is None.  Returns [B, len(rows), Hq].
    """
    q, k = _exact(q), _exact(k)
    b_, n, hq, d = _check_shapes(q, k, k)
    g = hq // k.shape[2]
    nb = _neighbour_fn(sigma, n, window, causal)
    scale = 1.0 / math.sqrt(d)
    rows = _rows_or_all(n, rows)
    out = np.empty((b_, rows.shape[0], hq), dtype=np.float64)
    for r, i in enumerate(rows):
        idx = nb(int(i))
        for b in range(b_):
            kj = k[b, idx].astype(np.float64)
            qi = q[b, i].astype(np.float64)
            for h in range(hq):
                out[b, r, h] = _row_probs(qi[h], kj[:, h // g, :], scale)[1]
    return out


# ----------------------------------------------------------------------------------------------
# Gradient contributions of one query row
# ----------------------------------------------------------------------------------------------

def _row_backward(q_i, k_b, v_b, idx, scale, dy_i, g_i):
    """Chain rule through one query row (all heads).

    q_i [Hq, d], dy_i [Hq, d], g_i [Hq] (gate values); k_b, v_b [n, Hkv, d]; idx int[m].
    Returns (dq_i [Hq, d], dk_rows [m, Hkv, d], dv_rows [m, Hkv, d], dg_i [Hq]); the key-side
    arrays are this row's contributions to the keys idx.
    """
    hq, d = q_i.shape
    hkv = k_b.shape[1]
    grp = hq // hkv
    kj = k_b[idx].astype(np.float64)
    vj = v_b[idx].astype(np.float64)
    dq_i = np.zeros((hq, d))
    dk_rows = np.zeros((idx.shape[0], hkv, d))
    dv_rows = np.zeros((idx.shape[0], hkv, d))
    dg_i = np.zeros(hq)
    for h in range(hq):
        kv = h // grp
        p, _ = _row_probs(q_i[h], kj[:, kv, :], scale)
        a = p @ vj[:, kv, :]                       # A_i
        da = g_i[h] * dy_i[h]                      # dA_i
        dg_i[h] = dy_i[h] @ a
        dv_rows[:, kv, :] += p[:, None] * da[None, :]
        dp = vj[:, kv, :] @ da                     # dP_j
        ds = p * (dp - p @ dp)                     # dS_j
        dq_i[h] = scale * (ds @ kj[:, kv, :])
        dk_rows[:, kv, :] += scale * ds[:, None] * q_i[h][None, :]
    return dq_i, dk_rows, dv_rows, dg_i


def _prep(q, k, v, dy, gate):
    q, k, v = _exact(q), _exact(k), _exact(v)
    b_, n, hq, d = _check_shapes(q, k, v)
    dy = _f64(dy)
    if dy.shape != q.shape:
        raise ValueError("dy must have the shape of q")
    gate = np.ones((b_, n, hq)) if gate is None else _f64(gate)
    if gate.shape != (b_, n, hq):
        raise ValueError("gate must be [B, n, Hq]")
    return q, k, v, dy, gate, b_, n, hq, d


def attention_backward(q, k, v, sigma, window: int, causal: bool, dy, gate=None):
    """Gradients of L = sum <dy, g * A> for A = SA (sigma given) or SWA (sigma None).

    Returns (dq [B,n,Hq,d], dk [B,n,Hkv,d], dv [B,n,Hkv,d], dg [B,n,Hq]) in float64.  With gate
    None the gate is 1 and dg is still <dy_i, A_i>.
    """
    if window < 1:
        raise ValueError("window must be >= 1")
    q, k, v, dy, gate, b_, n, hq, d = _prep(q, k, v, dy, gate)
    nb = _neighbour_fn(sigma, n, window, causal)
    scale = 1.0 / math.sqrt(d)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    dg = np.zeros((b_, n, hq))
    for i in range(n):
        idx = nb(i)
        for b in range(b_):
            dq_i, dk_r, dv_r, dg_i = _row_backward(q[b, i].astype(np.float64), k[b], v[b], idx,
                                                   scale, dy[b, i], gate[b, i])
            dq[b, i] = dq_i
            dg[b, i] = dg_i
            dk[b, idx] += dk_r                     # idx holds distinct keys
            dv[b, idx] += dv_r
    return dq, dk, dv, dg


def gated_backward(q, k, v, sigma, window: int, causal: bool, gates, dy):
    """Gradients of L = sum <dy, g_sa A_sa + g_swa A_swa> (same w and causal flag for both, R9).

    Returns (dq, dk, dv, dgates [2, B, n, Hq]).
    """
    gates = _f64(gates)
    a = attention_backward(q, k, v, sigma, window, causal, dy, gates[0])
    b = attention_backward(q, k, v, None, window, causal, dy, gates[1])
    return a[0] + b[0], a[1] + b[1], a[2] + b[2], np.stack([a[3], b[3]])


# ----------------------------------------------------------------------------------------------
# Sampled rows (large n): dQ and dg of given queries, dK and dV of given keys
# ----------------------------------------------------------------------------------------------

def attention_backward_query_rows(q, k, v, sigma, window: int, causal: bool, dy, gate,
                                  rows: Iterable[int]):
    """dq [B, len(rows), Hq, d] and dg [B, len(rows), Hq] of the given original query rows."""
    q, k, v, dy, gate, b_, n, hq, d = _prep(q, k, v, dy, gate)
    nb = _neighbour_fn(sigma, n, window, causal)
    scale = 1.0 / math.sqrt(d)
    rows = _rows_or_all(n, rows)
    dq = np.empty((b_, rows.shape[0], hq, d))
    dg = np.empty((b_, rows.shape[0], hq))
    for r, i in enumerate(rows):
        idx = nb(int(i))
        for b in range(b_):
            dq_i, _, _, dg_i = _row_backward(q[b, i].astype(np.float64), k[b], v[b], idx, scale,
                                             dy[b, i], gate[b, i])
            dq[b, r] = dq_i
            dg[b, r] = dg_i
    return dq, dg


def attending_queries(sigma, n: int, window: int, causal: bool, j: int) -> np.ndarray:
    """Original queries i whose neighbour set holds key j (SA with sigma, SWA without).

    Candidates come from the band (|slot(i) - slot(j)| <= w - 1); each is kept only if j is in
    its neighbour set, so the answer rests on the neighbour-set definition alone.
    """
    nb = _neighbour_fn(sigma, n, window, causal)
    if sigma is None:
        cand = range(max(0, j - window + 1), min(n, j + window))
    else:
        sigma = np.asarray(sigma)
        pj = int(inverse_permutation(sigma)[j])
        cand = (int(x) for x in sigma[max(0, pj - window + 1):min(n, pj + window)])
    return np.array(sorted(i for i in cand if j in set(nb(i).tolist())), dtype=np.int64)


def attention_backward_key_rows(q, k, v, sigma, window: int, causal: bool, dy, gate,
                                keys: Iterable[int]):
    """dk and dv [B, len(keys), Hkv, d] of the given original key rows.

    Sums the contributions of every query that attends to each key.
    """
    q, k, v, dy, gate, b_, n, hq, d = _prep(q, k, v, dy, gate)
    nb = _neighbour_fn(sigma, n, window, causal)
    scale = 1.0 / math.sqrt(d)
    keys = _rows_or_all(n, keys)
    hkv = k.shape[2]
    dk = np.zeros((b_, keys.shape[0], hkv, d))
    dv = np.zeros((b_, keys.shape[0], hkv, d))
    for r, j in enumerate(keys):
        for i in attending_queries(sigma, n, window, causal, int(j)):
            idx = nb(int(i))
            pos = int(np.nonzero(idx == j)[0][0])
            for b in range(b_):
                _, dk_r, dv_r, _ = _row_backward(q[b, i].astype(np.float64), k[b], v[b], idx,
                                                 scale, dy[b, i], gate[b, i])
                dk[b, r] += dk_r[pos]
                dv[b, r] += dv_r[pos]
    return dk, dv
