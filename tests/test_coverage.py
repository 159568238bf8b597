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


# ---- pins of the oracle's SA and gated modes (oracle only, no library code)
#
# [SA-ja] 理論的性質 (受容野の成長) describes the field of a position after l layers: everything
# reachable through the layers' neighbour sets.  The pins below fix coverage_by_layer in every
# mode from facts that do not use it: exact pair counts after one layer, full coverage when the
# window spans the sequence, and a second formulation as boolean matrix products of dense
# adjacency matrices built straight from the slot-space band of [SA-ja] 中核メカニズム step 2
# (not from the oracle's neighbour functions).

def _adjacency(n, w, causal, mode, sigma):
    """A[i, j] = 1 iff original position i attends to j in one layer.  SA: the band
    |p - q| <= w - 1 in slot space, and sigma[q] <= sigma[p] when causal; slot p holds token
    sigma[p].  SWA: the same with sigma = identity.  Gated: the union of the two."""
    idx = np.arange(n)
    band = np.abs(idx[:, None] - idx[None, :]) <= w - 1
    a = np.zeros((n, n), dtype=bool)
    if mode in ("sa", "gated"):
        a_pi = band & ((sigma[None, :] <= sigma[:, None]) if causal else True)
        a[np.ix_(sigma, sigma)] |= a_pi
    if mode in ("swa", "gated"):
        a |= band & ((idx[None, :] <= idx[:, None]) if causal else True)
    return a


def _coverage_by_matrix_products(n, w, seeds, mode, causal):
    reach = np.eye(n, dtype=np.int64)
    total = n * (n + 1) // 2 if causal else n * n
    out = []
    for seed in seeds:
        sigma = oracle.make_permutation(seed, n).astype(np.int64)
        reach = (_adjacency(n, w, causal, mode, sigma).astype(np.int64) @ reach > 0).astype(
            np.int64)
        out.append(reach.sum() / total)
    return np.array(out)


def _layer1_pairs(n, w, causal, mode, sigma):
    """Pairs after one layer, counted from the slot-space definition by brute force."""
    return int(_adjacency(n, w, causal, mode, sigma).sum())


@pytest.mark.parametrize("n,w", [(40, 1), (57, 6), (96, 13), (31, 31)])
def test_oracle_sa_one_layer_pair_count_closed_forms(n, w):
    """After one layer the field of i is its neighbour set, so the coverage is the number of
    attended pairs over the pair total.  Under the two-sided band: causal SA keeps, of each
    unordered in-band pair, exactly the direction that points back in original order, whatever
    sigma is, giving n*w - w(w-1)/2 pairs; non-causal SA keeps both, n(2w - 1) - w(w - 1)."""
    for seed in (1, 2, 3):
        causal = oracle.coverage_by_layer(n, w, [seed], "sa", causal=True)[0]
        assert causal == (n * w - w * (w - 1) // 2) / (n * (n + 1) // 2)
        nonc = oracle.coverage_by_layer(n, w, [seed], "sa", causal=False)[0]
        assert nonc == (n * (2 * w - 1) - w * (w - 1)) / (n * n)


@pytest.mark.parametrize("mode", ["sa", "swa", "gated"])
@pytest.mark.parametrize("causal", [True, False])
def test_oracle_full_window_covers_in_one_layer(mode, causal):
    for n, w in ((30, 30), (45, 60)):
        assert oracle.coverage_by_layer(n, w, [5], mode, causal)[0] == 1.0


def test_oracle_unit_window_never_grows():
    # w = 1: every neighbour set is the token itself, in every mode and layer
    for mode in ("sa", "swa", "gated"):
        for causal in (True, False):
            cov = oracle.coverage_by_layer(50, 1, [1, 2, 3], mode, causal)
            total = 50 * 51 / 2 if causal else 50 * 50
            assert np.all(cov == 50 / total)


@pytest.mark.parametrize("mode", ["sa", "swa", "gated"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("n,w", [(48, 3), (70, 5), (33, 9)])
def test_oracle_matches_boolean_matrix_products(mode, causal, n, w):
    seeds = [11 * n + l for l in range(4)]
    got = oracle.coverage_by_layer(n, w, seeds, mode, causal)
    ref = _coverage_by_matrix_products(n, w, seeds, mode, causal)
    assert np.array_equal(got, ref)


def test_oracle_gated_layer_one_is_the_union():
    """One gated layer attends to the union of the SA and SWA sets: its pair count lies between
    the larger of the two and their sum, and equals the brute-force union count."""
    n, w = 64, 7
    for causal in (True, False):
        sigma = oracle.make_permutation(9, n).astype(np.int64)
        total = n * (n + 1) // 2 if causal else n * n
        g = oracle.coverage_by_layer(n, w, [9], "gated", causal)[0] * total
        s = oracle.coverage_by_layer(n, w, [9], "sa", causal)[0] * total
        o = oracle.coverage_by_layer(n, w, [9], "swa", causal)[0] * total
        assert max(s, o) < g < s + o
        assert g == _layer1_pairs(n, w, causal, "gated", sigma)


# ---- planted mistakes in a copy of coverage_by_layer: each must fail one of the pins above

def _pins_fail(cov_fn):
    """Runs the pins above against cov_fn (same signature as coverage_by_layer); returns the
    names of the pins that fail."""
    failed = []
    n, w = 57, 6
    if cov_fn(n, w, [1], "sa", True)[0] != (n * w - w * (w - 1) // 2) / (n * (n + 1) // 2):
        failed.append("causal-layer1")
    if cov_fn(n, w, [1], "sa", False)[0] != (n * (2 * w - 1) - w * (w - 1)) / (n * n):
        failed.append("noncausal-layer1")
    for mode in ("sa", "swa", "gated"):
        for causal in (True, False):
            if cov_fn(30, 30, [5], mode, causal)[0] != 1.0:
                failed.append(f"full-window-{mode}-{causal}")
            seeds = [700 + l for l in range(4)]
            if not np.array_equal(cov_fn(48, 3, seeds, mode, causal),
                                  _coverage_by_matrix_products(48, 3, seeds, mode, causal)):
                failed.append(f"matrix-{mode}-{causal}")
    return failed


def _mutant(replacements):
    """A copy of oracle.coverage_by_layer with source substitutions applied."""
    import inspect
    import textwrap
    import oracle.coverage as C
    src = textwrap.dedent(inspect.getsource(C.coverage_by_layer))
    for old, new in replacements:
        assert old in src, old
        src = src.replace(old, new)
    ns = dict(vars(C))
    exec(compile(src, "<mutant>", "exec"), ns)
    return ns["coverage_by_layer"]


_MUTATIONS = {
    # one sigma for every layer instead of an independent draw per layer
    "one-sigma-for-all-layers": [("sigma = make_permutation(seed, n)",
                                  "sigma = make_permutation(seeds[0], n)")],
    # the gated layer intersects the two neighbour sets instead of taking their union
    "gated-intersection": [("nb |= set(swa_neighbours(n, window, causal, i).tolist())",
                            "nb = (nb & set(swa_neighbours(n, window, causal, i).tolist())) "
                            "if mode == 'gated' else (nb | set(swa_neighbours(n, window, "
                            "causal, i).tolist()))")],
    # R_l built from the partly updated R_l (in-place update) instead of R_{l-1}
    "in-place-update": [("acc |= fields[j]", "acc |= (new[j] if j < len(new) else fields[j])")],
    # the field of a position omits the position itself at the start
    "empty-start": [("fields = [{i} for i in range(n)]", "fields = [set() for i in range(n)]")],
    # the causal pair total counted as n^2
    "wrong-total": [("total = n * (n + 1) // 2 if causal else n * n", "total = n * n")],
    # the SA set of the gated layer taken non-causally
    "gated-sa-noncausal": [("nb |= set(sa_neighbours(sigma, window, causal, i, inv).tolist())",
                            "nb |= set(sa_neighbours(sigma, window, causal and mode == 'sa', i, "
                            "inv).tolist())")],
}


def test_unmutated_coverage_oracle_passes_the_pins():
    assert _pins_fail(oracle.coverage_by_layer) == []


@pytest.mark.parametrize("name", sorted(_MUTATIONS))
def test_each_planted_mistake_fails_a_pin(name):
    assert _pins_fail(_mutant(_MUTATIONS[name])) != [], name
