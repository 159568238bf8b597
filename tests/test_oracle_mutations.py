"""Planted mistakes in the oracle (on the CPU): each one must be caught by the pin battery.

The battery re-runs, in compact form, the checks of test_oracle_attention.py that rest on
something outside the oracle (torch SDPA special cases, exact pair counts, equivariance, the
causal no-future property, w = 1).  Every mutation below is a plausible slip -- an off-by-one
band, a strict causal test, sigma used in the wrong direction, the causal rule keyed on the
permuted slot, a dropped softmax scale, a swapped operand, a wrong GQA head map -- and the
test asserts that at least one pin fails under it.  The unmutated oracle passes the battery.
"""

import math

import numpy as np
import pytest
import torch

import oracle.attention as A
from oracle import make_permutation, inverse_permutation


def _rand(seed, B, n, Hq, Hkv, d):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, n, Hq, d)), r.standard_normal((B, n, Hkv, d)),
            r.standard_normal((B, n, Hkv, d)))


def _sdpa(q, k, v, mask=None, is_causal=False):
    g = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.repeat(k, g, axis=2)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(np.repeat(v, g, axis=2)).permute(0, 2, 1, 3)
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=m, is_causal=is_causal).permute(0, 2, 1, 3).numpy()


def _pin_identity_and_full_window(failed):
    n, w = 29, 5
    q, k, v = _rand(1, 1, n, 4, 2, 8)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    for causal in (False, True):
        mask = ((j <= i) & (j > i - w)) if causal else (np.abs(i - j) < w)
        y = A.sa_rows(q, k, v, np.arange(n, dtype=np.int32), w, causal)
        if np.abs(y - _sdpa(q, k, v, mask=mask)).max() > 1e-12:
            failed.append(f"identity-sdpa-{causal}")
        sigma = make_permutation(3, n)
        y = A.sa_rows(q, k, v, sigma, n, causal)
        if np.abs(y - _sdpa(q, k, v, is_causal=causal)).max() > 1e-12:
            failed.append(f"full-window-sdpa-{causal}")


def _pin_pair_count_and_no_future(failed):
    sigma = make_permutation(4, 40)
    inv = inverse_permutation(sigma)
    tot = sum(len(A.sa_neighbours(sigma, 6, True, t, inv)) for t in range(40))
    if tot != 40 * 6 - 15:
        failed.append("causal-pair-count")
    for t in range(40):
        nb = A.sa_neighbours(sigma, 6, True, t, inv)
        if len(nb) == 0 or nb.max() != t:
            failed.append("causal-no-future")
            break


def _pin_equivariance(failed):
    sigma = make_permutation(4, 40)
    q2, k2, v2 = _rand(5, 1, 40, 2, 1, 8)
    tau = make_permutation(6, 40)
    y = A.sa_rows(q2, k2, v2, sigma, 5, False)
    y2 = A.sa_rows(q2[:, tau], k2[:, tau], v2[:, tau], inverse_permutation(tau)[sigma], 5, False)
    if np.abs(y2 - y[:, tau]).max() > 1e-12:
        failed.append("equivariance")


def _pin_unit_window(failed):
    sigma = make_permutation(4, 40)
    q2, k2, v2 = _rand(5, 1, 40, 2, 1, 8)
    y1 = A.sa_rows(q2, k2, v2, sigma, 1, True)
    if np.abs(y1 - v2.repeat(2, axis=2)).max() > 1e-15:
        failed.append("unit-window")


def battery() -> list:
    """Names of the pins that FAIL for the oracle as currently bound in oracle.attention.

    A pin that raises (for instance on an empty neighbourhood) counts as failed.
    """
    failed = []
    for pin in (_pin_identity_and_full_window, _pin_pair_count_and_no_future, _pin_equivariance,
                _pin_unit_window):
        try:
            pin(failed)
        except Exception as e:  # noqa: BLE001 -- any crash is a caught mistake
            failed.append(f"{pin.__name__}: {type(e).__name__}")
    return failed


def test_unmutated_oracle_passes_battery():
    assert battery() == []


def _nb_off_by_one(sigma, window, causal, i, inv=None):
    sigma = np.asarray(sigma)
    n = sigma.shape[0]
    inv = inverse_permutation(sigma) if inv is None else inv
    p = int(inv[i])
    m = sigma[max(0, p - window):min(n - 1, p + window) + 1].astype(np.int64)
    return np.sort(m[m <= i] if causal else m)


def _nb_strict_causal(sigma, window, causal, i, inv=None):
    sigma = np.asarray(sigma)
    n = sigma.shape[0]
    inv = inverse_permutation(sigma) if inv is None else inv
    p = int(inv[i])
    m = sigma[max(0, p - window + 1):min(n - 1, p + window - 1) + 1].astype(np.int64)
    return np.sort(m[m < i] if causal else m)


def _nb_wrong_direction(sigma, window, causal, i, inv=None):
    sigma = np.asarray(sigma)
    n = sigma.shape[0]
    inv = inverse_permutation(sigma)
    p = int(sigma[i])                    # slot looked up through sigma instead of sigma^-1
    m = inv[max(0, p - window + 1):min(n - 1, p + window - 1) + 1].astype(np.int64)
    return np.sort(m[m <= i] if causal else m)


def _nb_causal_on_slot(sigma, window, causal, i, inv=None):
    sigma = np.asarray(sigma)
    n = sigma.shape[0]
    inv = inverse_permutation(sigma) if inv is None else inv
    p = int(inv[i])
    lo = max(0, p - window + 1)
    hi = p if causal else min(n - 1, p + window - 1)   # causal keyed on permuted position
    return np.sort(sigma[lo:hi + 1].astype(np.int64))


def _attend_no_scale(q_i, k_b, v_b, idx, scale):
    return _ORIG_ATTEND(q_i, k_b, v_b, idx, 1.0)


def _attend_k_for_v(q_i, k_b, v_b, idx, scale):
    return _ORIG_ATTEND(q_i, k_b, k_b, idx, scale)


def _attend_bad_gqa(q_i, k_b, v_b, idx, scale):
    hq, d = q_i.shape
    hkv = k_b.shape[1]
    out = np.empty((hq, d))
    for h in range(hq):
        kvh = h % hkv                     # interleaved instead of grouped head map
        s = scale * (k_b[idx][:, kvh, :] @ q_i[h])
        e = np.exp(s - s.max())
        out[h] = (e @ v_b[idx][:, kvh, :]) / e.sum()
    return out


_ORIG_ATTEND = A._attend_row


@pytest.mark.parametrize("name,target,fn", [
    ("band-off-by-one", "sa_neighbours", _nb_off_by_one),
    ("strict-causal", "sa_neighbours", _nb_strict_causal),
    ("sigma-direction", "sa_neighbours", _nb_wrong_direction),
    ("causal-on-permuted-slot", "sa_neighbours", _nb_causal_on_slot),
    ("dropped-scale", "_attend_row", _attend_no_scale),
    ("k-used-for-v", "_attend_row", _attend_k_for_v),
    ("gqa-head-map", "_attend_row", _attend_bad_gqa),
])
def test_planted_mistake_is_caught(monkeypatch, name, target, fn):
    monkeypatch.setattr(A, target, fn)
    failed = battery()
    assert failed, f"mutation {name} slipped through every pin"
