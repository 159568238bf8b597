"""CPU oracle for Stochastic Attention (SA), plain SWA and the gated SA+SWA combination.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously-correct reference the GPU
path is checked against.  It is imported by ``tests/``, by ``__graft_entry__.smoke()`` and
by the ``cpu_baseline`` leg of ``bench.py`` -- nothing in the product package
(``stochastic_sliding_window_amd``) imports it, and it imports nothing from there.

Everything is NumPy in float64 (the pages fix no precision), computed straight from the
definitions on the pages:

* permutation.py -- sigma ~ Uniform(S_n) per layer, drawn by a seeded Fisher-Yates shuffle
  fed by splitmix64 (the page asks only for a uniform permutation; the generator is the
  fixed, published one that both sides implement independently).
* attention.py   -- neighbour sets, SA / SWA / gated forward, and a second, permuted-space
  formulation of SA used to cross-check the first.
* backward.py    -- the gradients of those forwards (chain rule through the definition, one
  query row at a time), the rows' log-sum-exp, and sampled-row forms for large n.
* decode.py      -- one decode step over a KV cache (row t of causal SA over the full context).
* coverage.py    -- receptive-field growth over layers (sets, small n).
* gates.py       -- the gate projections g = sigmoid(x w + b) of the gated layer.

Sources (the pages):
  [SA-ja] "技術的概要：確率的アテンション" (gist.science/ja/paper/2604.00754) -- Stochastic
          Attention summary: 中核メカニズム (core mechanism) steps 1-3, 理論的性質 (theoretical
          properties), ゲート付き SA と SWA の組み合わせ (gated combination, the Y equation).
  [SA-ko] "기술 요약: 확률적 어텐션" (gist.science/ko/paper/2604.00754) -- the same summary in
          Korean; used to cross-check [SA-ja].
  [HYB]   notes on "Rethinking the Role of Efficient Attention in Hybrid Architectures"
          (notes.yuuk.io), section ハイブリッドアーキテクチャの定義 -- the SWA definition.

Pin status: every function here is pinned by CPU tests against facts the pages and the
mathematics fix (closed forms, library special cases, invariants, a published generator
test vector).  See tests/test_oracle_*.py.
"""

from .permutation import splitmix64_stream, fisher_yates, make_permutation, inverse_permutation
from .attention import (
    sa_neighbours,
    swa_neighbours,
    sa_rows,
    swa_rows,
    sa_forward,
    swa_forward,
    gated_forward,
    sa_forward_permuted_dense,
)
from .backward import (
    attention_lse_rows,
    attention_backward,
    gated_backward,
    attention_backward_query_rows,
    attention_backward_key_rows,
    attending_queries,
)
from .decode import sa_decode, swa_decode, gated_decode
from .coverage import coverage_by_layer
from .gates import gate_projection

__all__ = [
    "splitmix64_stream",
    "fisher_yates",
    "make_permutation",
    "inverse_permutation",
    "sa_neighbours",
    "swa_neighbours",
    "sa_rows",
    "swa_rows",
    "sa_forward",
    "swa_forward",
    "gated_forward",
    "sa_forward_permuted_dense",
    "attention_lse_rows",
    "attention_backward",
    "gated_backward",
    "attention_backward_query_rows",
    "attention_backward_key_rows",
    "attending_queries",
    "sa_decode",
    "swa_decode",
    "gated_decode",
    "coverage_by_layer",
    "gate_projection",
]
