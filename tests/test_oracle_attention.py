"""Pins of the oracle's SA / SWA / gated forward (CPU only, float64).

Each test checks the oracle against something other than itself:
* library special cases: with sigma = identity SA is the SWA of [HYB] (the w tokens up to and
  including t), which is torch's scaled_dot_product_attention with that band as a mask; with a
  window covering the whole sequence SA is plain full attention (causal or not) for ANY sigma;
* closed forms of the neighbourhood ([SA-ja] 中核メカニズム, random neighbourhood of expected
  size w and pairwise probability about w/n): exact per-row sizes (non-causal), the exact total
  pair count nw - w(w-1)/2 for every sigma (causal), and pair frequencies over many sigma;
* invariants: V = 1 gives Y = 1; w = 1 gives Y = V; relabelling equivariance; the gated output
  is linear in the gates ([SA-ja] gated combination equation);
* a second, permuted-space formulation written the way the page's three steps read.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import (sa_neighbours, swa_neighbours, sa_rows, swa_rows, sa_forward, swa_forward,
                    gated_forward, sa_forward_permuted_dense, make_permutation, inverse_permutation)


def _rand(seed, B, n, Hq, Hkv, d):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, n, Hq, d)), r.standard_normal((B, n, Hkv, d)),
            r.standard_normal((B, n, Hkv, d)))


def _sdpa(q, k, v, mask=None, is_causal=False):
    """torch SDPA in float64 on [B, n, H, d] numpy arrays (GQA expanded by repeat)."""
    B, n, Hq, d = q.shape
    g = Hq // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.repeat(k, g, axis=2)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(np.repeat(v, g, axis=2)).permute(0, 2, 1, 3)
    m = None if mask is None else torch.from_numpy(mask)
    y = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=is_causal)
    return y.permute(0, 2, 1, 3).numpy()


def _hyb_swa_mask(n, w, causal):
    # [HYB]: position t sees the w tokens up to and including itself; the non-causal form sees
    # w - 1 tokens on each side (R2).
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    if causal:
        return (j <= i) & (j > i - w)
    return np.abs(i - j) < w


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,w", [(37, 5), (64, 16), (50, 1), (33, 40)])
def test_identity_sigma_is_swa_and_sdpa(causal, n, w):
    q, k, v = _rand(n * 7 + w, 2, n, 4, 2, 8)
    ident = np.arange(n, dtype=np.int32)
    y_sa = sa_forward(q, k, v, ident, w, causal)
    y_swa = swa_forward(q, k, v, w, causal)
    y_lib = _sdpa(q, k, v, mask=_hyb_swa_mask(n, w, causal))
    np.testing.assert_allclose(y_sa, y_lib, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y_swa, y_lib, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,w", [(40, 40), (23, 100)])
def test_window_covering_sequence_is_full_attention(causal, n, w):
    q, k, v = _rand(99 + n, 1, n, 6, 3, 16)
    for seed in (1, 2, 3):
        sigma = make_permutation(seed, n)
        y = sa_forward(q, k, v, sigma, w, causal)
        y_lib = _sdpa(q, k, v, is_causal=causal)
        np.testing.assert_allclose(y, y_lib, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,w,B,Hq,Hkv", [(48, 6, 2, 4, 2), (61, 13, 1, 3, 1), (16, 3, 1, 2, 2)])
def test_original_space_equals_permuted_space(causal, n, w, B, Hq, Hkv):
    q, k, v = _rand(5 * n + w, B, n, Hq, Hkv, 8)
    for seed in (10, 11):
        sigma = make_permutation(seed, n)
        a = sa_forward(q, k, v, sigma, w, causal)
        b = sa_forward_permuted_dense(q, k, v, sigma, w, causal)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_row_sampling_matches_full():
    n = 70
    q, k, v = _rand(3, 2, n, 4, 1, 8)
    sigma = make_permutation(77, n)
    rows = [0, 5, 69, 33]
    full = sa_forward(q, k, v, sigma, 9, True)
    part = sa_rows(q, k, v, sigma, 9, True, rows)
    np.testing.assert_array_equal(full[:, rows], part)


@pytest.mark.parametrize("n,w", [(256, 16), (100, 7), (31, 31), (64, 1)])
def test_causal_total_pairs_exact_for_every_sigma(n, w):
    # Every in-band unordered pair {p, q}, p != q, is kept in exactly one direction (one of the two
    # tokens precedes the other in original order) and every token keeps itself, so the total is
    # n + sum_{t=1}^{w-1} (n - t) = n w - w (w - 1) / 2 -- the causal SWA pair count -- whatever
    # sigma is.
    for seed in range(5):
        sigma = make_permutation(seed, n)
        inv = inverse_permutation(sigma)
        tot = sum(len(sa_neighbours(sigma, w, True, i, inv)) for i in range(n))
        assert tot == n * w - w * (w - 1) // 2
        assert tot == sum(len(swa_neighbours(n, w, True, i)) for i in range(n))


@pytest.mark.parametrize("n,w", [(256, 16), (50, 9)])
def test_noncausal_neighbourhood_size_closed_form(n, w):
    sigma = make_permutation(123, n)
    inv = inverse_permutation(sigma)
    for i in range(n):
        p = int(inv[i])
        expect = min(p + w - 1, n - 1) - max(p - w + 1, 0) + 1
        nb = sa_neighbours(sigma, w, False, i, inv)
        assert len(nb) == expect
        assert i in nb
    tot = sum(len(sa_neighbours(sigma, w, False, i, inv)) for i in range(n))
    assert tot == n * (2 * w - 1) - w * (w - 1)


def test_pair_frequency_matches_closed_form_and_page():
    # [SA-ja] 中核メカニズム: any token pair is connected with probability about w/n.  Under the
    # band reading the exact probability that two distinct slots fall within w - 1 of each other
    # is P = (w - 1)(2n - w) / (n (n - 1)); causally only j < i can connect, so over ordered pairs
    # the connection rate is P / 2 ~= w / n.
    n, w, draws = 64, 8, 3000
    p_band = (w - 1) * (2 * n - w) / (n * (n - 1))
    hits_nc = 0
    hits_c = 0
    mean_size = np.zeros(n)
    pairs_nc = 0
    for seed in range(draws):
        sigma = make_permutation(50000 + seed, n)
        inv = inverse_permutation(sigma)
        # fixed probe pairs (i, j), i > j
        for (i, j) in ((40, 3), (63, 0), (10, 9)):
            hits_nc += j in sa_neighbours(sigma, w, False, i, inv)
            hits_c += j in sa_neighbours(sigma, w, True, i, inv)
            pairs_nc += 1
        for i in (0, 20, 63):
            mean_size[i] += len(sa_neighbours(sigma, w, True, i, inv))
    for hits in (hits_nc, hits_c):
        f = hits / pairs_nc
        sd = math.sqrt(p_band * (1 - p_band) / pairs_nc)
        assert abs(f - p_band) < 4 * sd, (f, p_band)
    # ordered-pair rate in the causal case is exactly P_band / 2 = (w-1)(2n-w) / (2n(n-1)), which
    # is w/n (the page's figure) up to relative terms of order 1/w and w/n
    assert abs(p_band / 2 - w / n) <= (w / n) * (1 / w + w / n)
    # causal E|N(i)| = 1 + P_band * i
    for i in (0, 20, 63):
        m = mean_size[i] / draws
        assert abs(m - (1 + p_band * i)) < 0.1 + 4 * math.sqrt(p_band * i / draws), (i, m)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_and_unit_window(causal):
    n = 45
    q, k, v = _rand(8, 1, n, 2, 2, 4)
    sigma = make_permutation(9, n)
    ones = np.ones_like(v)
    np.testing.assert_allclose(sa_forward(q, k, ones, sigma, 6, causal), 1.0, rtol=0, atol=1e-14)
    # w = 1: the band holds only the token itself, whatever sigma is
    np.testing.assert_allclose(sa_forward(q, k, v, sigma, 1, causal), v, rtol=0, atol=1e-15)


def test_zero_query_gives_uniform_average_over_neighbourhood():
    # Q = 0 makes every score equal, so Y[i] is the plain mean of V over N(i); with V one-hot over
    # the token index, Y[i, j] = 1/|N(i)| exactly when j is a neighbour.
    n, w = 24, 4
    q = np.zeros((1, n, 1, n))
    k = np.random.default_rng(0).standard_normal((1, n, 1, n))
    v = np.eye(n).reshape(1, n, 1, n)
    sigma = make_permutation(31, n)
    inv = inverse_permutation(sigma)
    for causal in (False, True):
        y = sa_forward(q, k, v, sigma, w, causal)[0, :, 0, :]
        for i in range(n):
            nb = sa_neighbours(sigma, w, causal, i, inv)
            row = np.zeros(n)
            row[nb] = 1.0 / len(nb)
            np.testing.assert_allclose(y[i], row, rtol=0, atol=1e-15)


def test_relabelling_equivariance_noncausal():
    # Relabel the tokens by tau: X'[i] = X[tau[i]].  With sigma' = tau^-1 o sigma the permuted
    # sequence is unchanged (X'[sigma'[p]] = X[sigma[p]]), so Y' = Y[tau].  This fixes the
    # direction of sigma (gather by sigma, scatter by sigma^-1).
    n, w = 40, 5
    q, k, v = _rand(4, 1, n, 2, 1, 8)
    sigma = make_permutation(5, n)
    tau = make_permutation(6, n)
    tau_inv = inverse_permutation(tau)
    sigma2 = tau_inv[sigma]
    y = sa_forward(q, k, v, sigma, w, False)
    y2 = sa_forward(q[:, tau], k[:, tau], v[:, tau], sigma2, w, False)
    np.testing.assert_allclose(y2, y[:, tau], rtol=0, atol=1e-13)
    # the flipped convention (scatter by sigma) is a different operator
    y_flip = sa_forward(q, k, v, inverse_permutation(sigma), w, False)
    assert np.abs(y_flip - y).max() > 1e-3


def test_gated_is_linear_in_gates():
    n, w, B, Hq, Hkv = 30, 4, 2, 4, 2
    q, k, v = _rand(12, B, n, Hq, Hkv, 8)
    sigma = make_permutation(13, n)
    r = np.random.default_rng(14)
    y_sa = sa_forward(q, k, v, sigma, w, True)
    y_swa = swa_forward(q, k, v, w, True)
    g = np.zeros((2, B, n, Hq))
    g[0] = 1.0
    np.testing.assert_allclose(gated_forward(q, k, v, sigma, w, True, g), y_sa, rtol=0, atol=0)
    g = np.zeros((2, B, n, Hq))
    g[1] = 1.0
    np.testing.assert_allclose(gated_forward(q, k, v, sigma, w, True, g), y_swa, rtol=0, atol=0)
    g = r.uniform(size=(2, B, n, Hq))
    want = g[0][..., None] * y_sa + g[1][..., None] * y_swa
    np.testing.assert_allclose(gated_forward(q, k, v, sigma, w, True, g), want, rtol=0, atol=1e-15)
    rows = [3, 29]
    np.testing.assert_allclose(gated_forward(q, k, v, sigma, w, True, g, rows), want[:, rows],
                               rtol=0, atol=1e-15)


def test_two_token_closed_form():
    # n = 2, w = 2, non-causal, one head, d = 1: each token sees both.  Softmax of two scores
    # s0, s1 gives weights 1/(1 + e^{s1 - s0}) and 1/(1 + e^{s0 - s1}).
    q = np.array([0.7, -1.3]).reshape(1, 2, 1, 1)
    k = np.array([0.2, 0.9]).reshape(1, 2, 1, 1)
    v = np.array([5.0, -2.0]).reshape(1, 2, 1, 1)
    for sigma in ([0, 1], [1, 0]):
        y = sa_forward(q, k, v, np.array(sigma, dtype=np.int32), 2, False)[0, :, 0, 0]
        for i in range(2):
            s0, s1 = q[0, i, 0, 0] * 0.2, q[0, i, 0, 0] * 0.9      # scale 1/sqrt(1) = 1
            a0 = 1 / (1 + math.exp(s1 - s0))
            assert abs(y[i] - (a0 * 5.0 + (1 - a0) * -2.0)) < 1e-14
        # causal: token 0 sees only itself, token 1 sees both
        yc = sa_forward(q, k, v, np.array(sigma, dtype=np.int32), 2, True)[0, :, 0, 0]
        assert yc[0] == 5.0
        s0, s1 = q[0, 1, 0, 0] * 0.2, q[0, 1, 0, 0] * 0.9
        a0 = 1 / (1 + math.exp(s1 - s0))
        assert abs(yc[1] - (a0 * 5.0 + (1 - a0) * -2.0)) < 1e-14


def test_causal_never_sees_future():
    n, w = 80, 20
    for seed in range(4):
        sigma = make_permutation(seed, n)
        inv = inverse_permutation(sigma)
        for i in range(n):
            nb = sa_neighbours(sigma, w, True, i, inv)
            assert nb.max() == i          # self is always there, nothing after it
        # a future-token perturbation leaves causal outputs before it unchanged
    q, k, v = _rand(1, 1, n, 1, 1, 4)
    sigma = make_permutation(2, n)
    y = sa_forward(q, k, v, sigma, w, True)
    k2, v2 = k.copy(), v.copy()
    k2[:, 60:] += 3.0
    v2[:, 60:] -= 2.0
    y2 = sa_forward(q, k2, v2, sigma, w, True)
    np.testing.assert_array_equal(y[:, :60], y2[:, :60])
