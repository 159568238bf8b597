"""Pins of the oracle's gradients (CPU).

The backward pass is fixed by the forward definition ([SA-ja] 中核メカニズム, 理論的性質, and the
gated equation), so each pin checks the oracle's gradients against something that does not
reuse its backward code:

* central finite differences of the forward (itself pinned in test_oracle_attention.py);
* torch.autograd through torch's scaled_dot_product_attention on a dense mask made from the
  neighbour sets;
* closed forms that follow from the softmax and the bilinear scores;
* the log-sum-exp against torch.logsumexp and against log |N(i)| for zero queries.

The planted-mistake battery at the end checks that every plausible slip in the row backward
fails at least one of these pins.
"""

import math

import numpy as np
import pytest
import torch

import oracle.attention as A
import oracle.backward as Bw
from oracle import make_permutation, inverse_permutation


def _inputs(seed, B, n, Hq, Hkv, d):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, n, Hq, d)), r.standard_normal((B, n, Hkv, d)),
            r.standard_normal((B, n, Hkv, d)), r.standard_normal((B, n, Hq, d)),
            r.uniform(0.05, 0.95, (B, n, Hq)))


def _forward(q, k, v, sigma, w, causal):
    if sigma is None:
        return A.swa_rows(q, k, v, w, causal)
    return A.sa_rows(q, k, v, sigma, w, causal)


def _finite_difference_error(q, k, v, sigma, w, causal, dy, g, grads, h=1e-6):
    """max |central difference - oracle gradient| over every coordinate of q, k, v and g."""
    def loss():
        return float((dy * g[..., None] * _forward(q, k, v, sigma, w, causal)).sum())
    err = 0.0
    for arr, grad in zip((q, k, v, g), grads):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss()
            arr[idx] = old - h
            lm = loss()
            arr[idx] = old
            err = max(err, abs((lp - lm) / (2 * h) - grad[idx]))
    return err


CASES = [(sa, causal) for sa in (True, False) for causal in (False, True)]


@pytest.mark.parametrize("sa,causal", CASES)
def test_gradients_match_finite_differences(sa, causal):
    B, n, Hq, Hkv, d, w = 1, 11, 4, 2, 8, 3
    q, k, v, dy, g = _inputs(10 + 2 * sa + causal, B, n, Hq, Hkv, d)
    sigma = make_permutation(5, n) if sa else None
    grads = Bw.attention_backward(q, k, v, sigma, w, causal, dy, g)
    assert _finite_difference_error(q, k, v, sigma, w, causal, dy, g, grads) < 1e-7


def test_gated_gradients_match_finite_differences():
    B, n, Hq, Hkv, d, w = 2, 9, 2, 1, 4, 3
    q, k, v, dy, _ = _inputs(21, B, n, Hq, Hkv, d)
    gates = np.random.default_rng(22).uniform(0.05, 0.95, (2, B, n, Hq))
    sigma = make_permutation(23, n)
    dq, dk, dv, dgates = Bw.gated_backward(q, k, v, sigma, w, True, gates, dy)

    def loss():
        return float((dy * A.gated_forward(q, k, v, sigma, w, True, gates)).sum())
    h = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv), (gates, dgates)):
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = loss()
            arr[idx] = old - h
            lm = loss()
            arr[idx] = old
            assert abs((lp - lm) / (2 * h) - grad[idx]) < 1e-7


def _dense_mask(sigma, n, w, causal):
    """mask[i, j] = j in N(i), built from the (pinned) neighbour sets."""
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        idx = (A.swa_neighbours(n, w, causal, i) if sigma is None
               else A.sa_neighbours(sigma, w, causal, i))
        m[i, idx] = True
    return m


def _autograd(q, k, v, sigma, w, causal, dy, g):
    """Gradients of sum <dy, g * SDPA(q, k, v, mask)> by torch.autograd, float64 on the CPU."""
    grp = q.shape[2] // k.shape[2]
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(k, requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    mask = torch.from_numpy(_dense_mask(sigma, q.shape[1], w, causal))
    y = torch.nn.functional.scaled_dot_product_attention(
        qt.permute(0, 2, 1, 3), kt.repeat_interleave(grp, dim=2).permute(0, 2, 1, 3),
        vt.repeat_interleave(grp, dim=2).permute(0, 2, 1, 3), attn_mask=mask).permute(0, 2, 1, 3)
    (torch.from_numpy(dy) * gt[..., None] * y).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), gt.grad.numpy()


@pytest.mark.parametrize("sa,causal", CASES)
def test_gradients_match_torch_autograd_of_sdpa(sa, causal):
    B, n, Hq, Hkv, d, w = 2, 37, 8, 2, 16, 6
    q, k, v, dy, g = _inputs(30 + 2 * sa + causal, B, n, Hq, Hkv, d)
    sigma = make_permutation(31, n) if sa else None
    ours = Bw.attention_backward(q, k, v, sigma, w, causal, dy, g)
    ref = _autograd(q, k, v, sigma, w, causal, dy, g)
    for a, b in zip(ours, ref):
        assert np.abs(a - b).max() < 1e-11


@pytest.mark.parametrize("sa,causal", CASES)
def test_closed_forms(sa, causal):
    B, n, Hq, Hkv, d, w = 1, 64, 4, 2, 16, 8
    q, k, v, dy, g = _inputs(40 + 2 * sa + causal, B, n, Hq, Hkv, d)
    sigma = make_permutation(41, n) if sa else None
    dq, dk, dv, dg = Bw.attention_backward(q, k, v, sigma, w, causal, dy, g)
    grp = Hq // Hkv
    # every softmax row sums to 1: the dV rows of a KV head sum to the gated upstream gradient of
    # its query heads
    gdy = (g[..., None] * dy).reshape(B, n, Hkv, grp, d).sum(axis=(1, 3))
    assert np.abs(dv.sum(axis=1) - gdy).max() < 1e-12
    # adding one vector to every key of a head leaves every row unchanged
    assert np.abs(dk.sum(axis=1)).max() < 1e-12
    # scores are bilinear in Q and K: scaling Q or K by the same factor changes them alike
    assert abs((dq * q).sum() - (dk * k).sum()) < 1e-11
    # dg is the upstream gradient against the attention output
    y = _forward(q, k, v, sigma, w, causal)
    assert np.abs(dg - (dy * y).sum(axis=-1)).max() < 1e-12


def test_equal_value_rows_give_zero_score_gradients():
    B, n, Hq, Hkv, d, w = 1, 50, 4, 2, 8, 7
    q, k, _, dy, g = _inputs(50, B, n, Hq, Hkv, d)
    v = np.broadcast_to(np.random.default_rng(51).standard_normal((1, 1, Hkv, d)),
                        (B, n, Hkv, d)).copy()
    dq, dk, dv, _ = Bw.attention_backward(q, k, v, make_permutation(52, n), w, True, dy, g)
    assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
    assert np.abs(dv).max() > 0.1


@pytest.mark.parametrize("sa,causal", CASES)
def test_lse_matches_torch_logsumexp(sa, causal):
    B, n, Hq, Hkv, d, w = 2, 40, 4, 1, 8, 5
    q, k, _, _, _ = _inputs(60, B, n, Hq, Hkv, d)
    sigma = make_permutation(61, n) if sa else None
    lse = Bw.attention_lse_rows(q, k, sigma, w, causal)
    mask = torch.from_numpy(_dense_mask(sigma, n, w, causal))
    s = torch.einsum("bihd,bjd->bhij", torch.from_numpy(q), torch.from_numpy(k[:, :, 0])) / math.sqrt(d)
    ref = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1).permute(0, 2, 1).numpy()
    assert np.abs(lse - ref).max() < 1e-12


def test_lse_of_zero_queries_counts_the_neighbours():
    n, w = 53, 6
    sigma = make_permutation(62, n)
    inv = inverse_permutation(sigma)
    k = np.random.default_rng(63).standard_normal((1, n, 1, 4))
    lse = Bw.attention_lse_rows(np.zeros((1, n, 2, 4)), k, sigma, w, True)
    for i in range(n):
        assert lse[0, i, 0] == pytest.approx(math.log(len(A.sa_neighbours(sigma, w, True, i, inv))),
                                             abs=1e-14)
    # causal pair count of the reading: n w - w (w - 1) / 2
    assert round(float(np.exp(lse[0, :, 1]).sum())) == n * w - w * (w - 1) // 2


@pytest.mark.parametrize("sa", [True, False])
def test_sampled_rows_equal_the_full_backward(sa):
    B, n, Hq, Hkv, d, w = 2, 40, 4, 2, 8, 5
    q, k, v, dy, g = _inputs(70, B, n, Hq, Hkv, d)
    sigma = make_permutation(71, n) if sa else None
    dq, dk, dv, dg = Bw.attention_backward(q, k, v, sigma, w, True, dy, g)
    rows = [0, 3, 17, 39]
    sq, sg = Bw.attention_backward_query_rows(q, k, v, sigma, w, True, dy, g, rows)
    assert np.abs(sq - dq[:, rows]).max() < 1e-13 and np.abs(sg - dg[:, rows]).max() < 1e-13
    sk, sv = Bw.attention_backward_key_rows(q, k, v, sigma, w, True, dy, g, rows)
    assert np.abs(sk - dk[:, rows]).max() < 1e-13 and np.abs(sv - dv[:, rows]).max() < 1e-13


def test_attending_queries_inverts_the_neighbour_sets():
    n, w = 45, 6
    sigma = make_permutation(72, n)
    for s in (sigma, None):
        for causal in (False, True):
            m = _dense_mask(s, n, w, causal)
            for j in range(n):
                assert Bw.attending_queries(s, n, w, causal, j).tolist() == np.nonzero(m[:, j])[0].tolist()


# ---- planted mistakes --------------------------------------------------------------------------

def _mutant(kind):
    def row_backward(q_i, k_b, v_b, idx, scale, dy_i, g_i):
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
            kv = h % hkv if kind == "gqa-map" else h // grp
            s = scale * (kj[:, kv, :] @ q_i[h])
            e = np.exp(s - s.max())
            p = e / e.sum()
            a = p @ vj[:, kv, :]
            da = dy_i[h] if kind == "ungated-da" else g_i[h] * dy_i[h]
            dg_i[h] = dy_i[h] @ a
            dv_rows[:, kv, :] += p[:, None] * (dy_i[h] if kind == "ungated-dv" else da)[None, :]
            dp = vj[:, kv, :] @ da
            if kind == "no-delta":
                ds = p * dp
            elif kind == "delta-sign":
                ds = p * (dp + p @ dp)
            else:
                ds = p * (dp - p @ dp)
            sc = 1.0 if kind == "no-scale" else scale
            dq_i[h] = sc * (ds @ kj[:, kv, :]) if kind != "dq-uses-v" else sc * (ds @ vj[:, kv, :])
            dk_rows[:, kv, :] += sc * ds[:, None] * (dy_i[h] if kind == "dk-uses-dy" else q_i[h])[None, :]
        return dq_i, dk_rows, dv_rows, dg_i
    return row_backward


def _battery_fails():
    failed = []
    B, n, Hq, Hkv, d, w = 1, 8, 4, 2, 4, 3
    q, k, v, dy, g = _inputs(80, B, n, Hq, Hkv, d)
    sigma = make_permutation(81, n)
    grads = Bw.attention_backward(q, k, v, sigma, w, True, dy, g)
    if _finite_difference_error(q, k, v, sigma, w, True, dy, g, grads) > 1e-7:
        failed.append("finite-differences")
    q, k, v, dy, g = _inputs(82, 1, 24, 4, 2, 8)
    ours = Bw.attention_backward(q, k, v, make_permutation(83, 24), 5, False, dy, g)
    ref = _autograd(q, k, v, make_permutation(83, 24), 5, False, dy, g)
    if max(np.abs(a - b).max() for a, b in zip(ours, ref)) > 1e-11:
        failed.append("autograd")
    return failed


def test_unmutated_backward_passes_the_battery():
    assert _battery_fails() == []


@pytest.mark.parametrize("kind", ["gqa-map", "ungated-da", "ungated-dv", "no-delta", "delta-sign",
                                  "no-scale", "dq-uses-v", "dk-uses-dy"])
def test_planted_mistake_is_caught(kind, monkeypatch):
    monkeypatch.setattr(Bw, "_row_backward", _mutant(kind))
    assert _battery_fails() != []
