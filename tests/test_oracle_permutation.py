"""Pins of the oracle's permutation generator (CPU only).

What fixes the answer here is not the oracle itself:
* the published splitmix64 test vector (tests/golden/splitmix64.txt);
* hand-worked Fisher-Yates shuffles from that vector (tests/golden/fisher_yates_small.txt);
* the page's requirement sigma ~ Uniform(S_n) ([SA-ja] 中核メカニズム step 1): a chi-square
  test over all 24 permutations of 4 items and over first-slot marginals;
* sigma^-1 o sigma = sigma o sigma^-1 = id ([SA-ja] step 3).
"""

import numpy as np
import pytest

from conftest import read_golden
from oracle import splitmix64_stream, fisher_yates, make_permutation, inverse_permutation


def test_splitmix64_published_vector():
    lines = read_golden("splitmix64.txt")
    assert lines[0].startswith("seed ")
    seed = int(lines[0].split()[1])
    expected = [int(x) for x in lines[1:]]
    assert splitmix64_stream(seed, len(expected)) == expected


def test_fisher_yates_hand_worked():
    for ln in read_golden("fisher_yates_small.txt"):
        vals = [int(x) for x in ln.split()]
        seed, n, sigma = vals[0], vals[1], vals[2:]
        assert fisher_yates(seed, n) == sigma


@pytest.mark.parametrize("n", [0, 1, 2, 7, 256, 4096])
def test_permutation_is_bijection_and_inverse(n):
    for seed in (0, 1, 2024, 2**63 + 5):
        s = make_permutation(seed, n)
        assert s.dtype == np.int32 and s.shape == (n,)
        assert sorted(s.tolist()) == list(range(n))
        if n == 0:
            continue
        inv = inverse_permutation(s)
        assert np.array_equal(inv[s], np.arange(n))
        assert np.array_equal(s[inv], np.arange(n))


def test_inverse_rejects_non_permutation():
    with pytest.raises(ValueError):
        inverse_permutation(np.array([0, 0, 2], dtype=np.int32))


def test_uniform_over_s4_chi_square():
    # 24 equally likely outcomes; 48,000 seeds -> 2,000 expected per cell.
    counts = {}
    trials = 48000
    for seed in range(trials):
        key = tuple(fisher_yates(seed, 4))
        counts[key] = counts.get(key, 0) + 1
    assert len(counts) == 24
    exp = trials / 24
    chi2 = sum((c - exp) ** 2 / exp for c in counts.values())
    # chi-square, 23 degrees of freedom: P(X > 49.73) = 0.001
    assert chi2 < 49.73, chi2


def test_first_slot_marginal_uniform():
    n, trials = 16, 16000
    counts = np.zeros(n)
    last = np.zeros(n)
    for seed in range(10**6, 10**6 + trials):
        s = fisher_yates(seed, n)
        counts[s[0]] += 1
        last[s[-1]] += 1
    exp = trials / n
    for c in (counts, last):
        chi2 = float(((c - exp) ** 2 / exp).sum())
        # 15 degrees of freedom: P(X > 37.70) = 0.001
        assert chi2 < 37.70, chi2


def test_layers_draw_independent_permutations():
    # [SA-ja] step 1: a fresh sigma per layer -> different seeds give different permutations.
    a = make_permutation(4001, 4096)
    b = make_permutation(4002, 4096)
    assert not np.array_equal(a, b)
    # agreement on a slot is 1/n per slot for independent uniform draws
    assert (a == b).sum() < 20
