"""Receptive-field coverage (CPU): the library's host tool against the set-based oracle, the
oracle against the SWA closed form, and the growth the pages describe ([SA-ja] 理論的性質,
受容野の成長: linear for SWA, O(log_w n) layers to full coverage for SA)."""

import numpy as np
import pytest

import oracle
import stochastic_sliding_window_amd as ssw


def _swa_closed_form(n, w, layers):
    # causal SWA: R_l(i) = [max(0, i - l (w - 1)), i]
    i = np.arange(n)
    return np.array([np.minimum(i + 1, l * (w - 1) + 1).sum() / (n * (n + 1) / 2)
                     for l in range(1, layers + 1)])


@pytest.mark.parametrize("n,w", [(50, 4), (97, 7), (64, 1)])
def test_oracle_swa_matches_closed_form(n, w):
    got = oracle.coverage_by_layer(n, w, range(6), "swa")
    assert np.abs(got - _swa_closed_form(n, w, 6)).max() < 1e-15


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("mode", ["sa", "swa", "gated"])
@pytest.mark.parametrize("n,w", [(80, 4), (131, 9), (40, 1), (33, 50)])
def test_library_tool_matches_oracle(mode, n, w, causal):
    seeds = [7 * n + l for l in range(5)]
    assert np.array_equal(ssw.receptive_field_coverage(n, w, seeds, mode, causal),
                          oracle.coverage_by_layer(n, w, seeds, mode, causal))


def test_oracle_noncausal_swa_closed_form():
    # |i - j| <= l (w - 1): the field of i after l layers is that interval cut to [0, n)
    n, w = 60, 5
    got = oracle.coverage_by_layer(n, w, range(4), "swa", causal=False)
    i = np.arange(n)
    ref = [(np.minimum(n - 1, i + l * (w - 1)) - np.maximum(0, i - l * (w - 1)) + 1).sum() / n**2
           for l in range(1, 5)]
    assert np.abs(got - np.array(ref)).max() < 1e-15


def test_full_window_covers_in_one_layer_and_unit_window_never_grows():
    assert ssw.receptive_field_coverage(200, 200, [1], "sa")[0] == 1.0
    cov = ssw.receptive_field_coverage(200, 1, [1, 2, 3], "sa")
    assert np.allclose(cov, 200 / (200 * 201 / 2))


def _first_full(cov):
    return int(np.argmax(cov >= 1.0)) + 1 if (cov >= 1.0).any() else None


@pytest.mark.parametrize("n,w", [(4096, 16), (4096, 64), (1024, 8)])
def test_full_coverage_in_logarithmically_many_layers(n, w):
    """Non-causal SA and the causal gated layer cover the sequence within a couple of layers of
    log_w n; SWA after as many layers covers only its linearly grown window."""
    seeds = list(range(1, 9))
    log_w_n = np.log(n) / np.log(w)
    sa = ssw.receptive_field_coverage(n, w, seeds, "sa", causal=False)
    gated = ssw.receptive_field_coverage(n, w, seeds, "gated", causal=True)
    swa = ssw.receptive_field_coverage(n, w, seeds, "swa", causal=True)
    assert _first_full(sa) is not None and _first_full(sa) <= np.ceil(log_w_n) + 2
    assert _first_full(gated) is not None and _first_full(gated) <= np.ceil(log_w_n) + 2
    assert _first_full(swa) is None and swa[-1] < 8 * w * 2 / n + 1e-9
    assert np.all(np.diff(sa) >= 0) and np.all(np.diff(gated) >= 0)
