"""Pins of the oracle's decode step (CPU).

Reading R20: decoding token t is row t of causal SA over the full context, with one sigma per
layer drawn over n_max.  The pins check the decode step against things it does not share code
paths with where possible: the pinned forward's row t, torch SDPA over the cache prefix, the
identity and full-window reductions, and the rule that nothing past t is read.
"""

import math

import numpy as np
import pytest
import torch

import oracle.attention as A
import oracle.decode as Dc
from oracle import make_permutation


def _cache(seed, B, n, Hq, Hkv, d):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, n, Hq, d)), r.standard_normal((B, n, Hkv, d)),
            r.standard_normal((B, n, Hkv, d)))


def test_decode_row_equals_forward_row():
    B, n, Hq, Hkv, d, w = 2, 70, 4, 2, 8, 9
    q, k, v = _cache(1, B, n, Hq, Hkv, d)
    sigma = make_permutation(2, n)
    y = A.sa_rows(q, k, v, sigma, w, True)
    for t in (0, 1, 8, 35, 69):
        pos = np.array([t, n - 1 - t])
        qd = np.stack([q[0, t], q[1, n - 1 - t]])
        yd = Dc.sa_decode(qd, k, v, sigma, w, pos)
        assert np.abs(yd[0] - y[0, t]).max() < 1e-13
        assert np.abs(yd[1] - y[1, n - 1 - t]).max() < 1e-13


def _sdpa_prefix(q_t, k, v, lo, hi):
    """torch SDPA of one query over cache rows [lo, hi] (fp64)."""
    grp = q_t.shape[0] // k.shape[1]
    qt = torch.from_numpy(q_t)[:, None, :]                                 # [Hq, 1, d]
    kk = torch.from_numpy(np.repeat(k[lo:hi + 1], grp, axis=1)).permute(1, 0, 2)
    vv = torch.from_numpy(np.repeat(v[lo:hi + 1], grp, axis=1)).permute(1, 0, 2)
    return torch.nn.functional.scaled_dot_product_attention(qt, kk, vv)[:, 0].numpy()


@pytest.mark.parametrize("w", [1, 5, 16])
def test_swa_step_is_sdpa_over_the_last_w_positions(w):
    B, n, Hq, Hkv, d = 3, 40, 8, 2, 16
    q, k, v = _cache(3, B, n, Hq, Hkv, d)
    pos = np.array([0, 7, 39])
    qd = q[np.arange(B), pos]
    y = Dc.swa_decode(qd, k, v, w, pos)
    for b in range(B):
        ref = _sdpa_prefix(qd[b], k[b], v[b], max(0, pos[b] - w + 1), pos[b])
        assert np.abs(y[b] - ref).max() < 1e-12


def test_full_window_sa_step_is_causal_attention_for_any_sigma():
    B, n, Hq, Hkv, d = 2, 33, 4, 4, 8
    q, k, v = _cache(4, B, n, Hq, Hkv, d)
    pos = np.array([20, 32])
    qd = q[np.arange(B), pos]
    for seed in (5, 6):
        y = Dc.sa_decode(qd, k, v, make_permutation(seed, n), n, pos)
        for b in range(B):
            assert np.abs(y[b] - _sdpa_prefix(qd[b], k[b], v[b], 0, pos[b])).max() < 1e-12


def test_identity_sigma_reduces_to_swa():
    B, n, Hq, Hkv, d, w = 2, 50, 4, 1, 8, 7
    q, k, v = _cache(7, B, n, Hq, Hkv, d)
    pos = np.array([3, 44])
    qd = q[np.arange(B), pos]
    a = Dc.sa_decode(qd, k, v, np.arange(n, dtype=np.int32), w, pos)
    assert np.abs(a - Dc.swa_decode(qd, k, v, w, pos)).max() < 1e-14


def test_decode_never_reads_past_t():
    B, n, Hq, Hkv, d, w = 1, 64, 2, 1, 8, 12
    q, k, v = _cache(8, B, n, Hq, Hkv, d)
    sigma = make_permutation(9, n)
    for t in (0, 10, 40):
        pos = np.array([t])
        qd = q[:, t]
        y = Dc.gated_decode(qd, k, v, sigma, w, pos, np.full((2, 1, Hq), 0.5))
        k2, v2 = k.copy(), v.copy()
        k2[:, t + 1:] = np.nan
        v2[:, t + 1:] = np.nan
        y2 = Dc.gated_decode(qd, k2, v2, sigma, w, pos, np.full((2, 1, Hq), 0.5))
        assert np.array_equal(y, y2)


def test_gates_are_linear():
    B, n, Hq, Hkv, d, w = 2, 30, 4, 2, 8, 5
    q, k, v = _cache(10, B, n, Hq, Hkv, d)
    sigma = make_permutation(11, n)
    pos = np.array([29, 12])
    qd = q[np.arange(B), pos]
    one, zero = np.ones((B, Hq)), np.zeros((B, Hq))
    assert np.abs(Dc.gated_decode(qd, k, v, sigma, w, pos, np.stack([one, zero])) -
                  Dc.sa_decode(qd, k, v, sigma, w, pos)).max() < 1e-15
    assert np.abs(Dc.gated_decode(qd, k, v, sigma, w, pos, np.stack([zero, one])) -
                  Dc.swa_decode(qd, k, v, w, pos)).max() < 1e-15


def test_bad_positions_rejected():
    q, k, v = _cache(12, 1, 10, 2, 1, 4)
    with pytest.raises(ValueError):
        Dc.swa_decode(q[:, 0], k, v, 3, np.array([10]))
