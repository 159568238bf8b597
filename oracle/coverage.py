"""Receptive-field growth over layers of SA / SWA / gated SA+SWA (oracle).
TEST INFRASTRUCTURE ONLY.

[SA-ja] 理論的性質 (受容野の成長) compares the two operators.  SWA's receptive field grows
linearly with depth, so it needs O(n/w) layers to cover the sequence.  SA draws an independent
permutation per layer, and the page states that full coverage then takes O(log_w n) layers.

Definitions.  Layer l has permutation sigma_l and neighbour sets N_l(i), which are those of the
forward oracle: SA, SWA, or their union for the gated layer, causal or not.  Then:
    R_0(i) = {i},    R_l(i) = union over j in N_l(i) of R_{l-1}(j).
The coverage after l layers is sum_i |R_l(i)| divided by the number of pairs (sum_i (i + 1) when
causal, n^2 otherwise): the share of pairs whose information has reached i.  Plain Python sets,
for small n only.

Pins (tests/test_coverage.py), none of which calls this function's helpers:
  * SWA closed forms: causal R_l(i) = [max(0, i - l (w - 1)), i], non-causal the interval
    |i - j| <= l (w - 1) cut to [0, n);
  * one SA layer: exactly n w - w (w - 1) / 2 attended pairs when causal (each unordered
    in-band pair points back in original order one way, whatever sigma is) and
    n (2 w - 1) - w (w - 1) when not;
  * a window spanning the sequence covers everything after one layer, a unit window never grows;
  * every mode over four layers equals a second formulation: boolean products of dense
    adjacency matrices built from the slot-space band itself;
  * planted mistakes (one sigma for all layers, an intersection for the gated layer, an
    in-place update, a wrong start, a wrong pair total) each fail one of these.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .attention import sa_neighbours, swa_neighbours
from .permutation import inverse_permutation, make_permutation


def coverage_by_layer(n: int, window: int, seeds: Sequence[int], mode: str,
                      causal: bool = True) -> np.ndarray:
    """Coverage after each of len(seeds) layers; mode 'sa', 'swa' or 'gated' (SA and SWA union).

    Layer l uses sigma = make_permutation(seeds[l], n) (ignored for 'swa').  The denominator is
    the number of pairs j <= i when causal, n^2 otherwise."""
    if mode not in ("sa", "swa", "gated"):
        raise ValueError(mode)
    fields = [{i} for i in range(n)]
    total = n * (n + 1) // 2 if causal else n * n
    out = []
    for seed in seeds:
        sigma = make_permutation(seed, n)
        inv = inverse_permutation(sigma)
        new = []
        for i in range(n):
            nb = set()
            if mode in ("sa", "gated"):
                nb |= set(sa_neighbours(sigma, window, causal, i, inv).tolist())
            if mode in ("swa", "gated"):
                nb |= set(swa_neighbours(n, window, causal, i).tolist())
            acc = set()
            for j in nb:
                acc |= fields[j]
            new.append(acc)
        fields = new
        out.append(sum(len(f) for f in fields) / total)
    return np.array(out)
