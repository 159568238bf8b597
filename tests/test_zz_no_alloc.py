"""The gated layer's backward that allocates nothing (ssw_gated_sa_swa_backward_noalloc, Delta in
the library's own device array) against the entry point that takes the caller's delta buffer
(ssw_gated_sa_swa_backward): the same gradients, bit for bit, on two calls in a row, the second
with a smaller input -- the array keeps the first call's contents, and the second call must not
depend on them.  Bit equality is stricter than the gradients' bar (1.5e-2 x max |oracle|): both
calls run the same kernels on the same values."""

import sys

import pytest
import torch

import oracle
import stochastic_sliding_window_amd as ssw
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(seed, B, n, Hq, Hkv, d, w, causal):
    print(f"no-alloc backward: B{B} n{n} Hq{Hq} Hkv{Hkv} d{d} w{w} causal={causal}",
          file=sys.stderr, flush=True)
    q, k, v = (t.to(DEV) for t in synth.qkv(seed, B, n, Hq, Hkv, d, "bf16"))
    g = synth.gates(seed, B, n, Hq).to(DEV)
    dy = synth.upstream_grad(seed, B, n, Hq, d, "bf16").to(DEV)
    sig_h = ssw.make_permutation(seed + 1, n)
    assert (sig_h == oracle.make_permutation(seed + 1, n)).all()
    sig = torch.from_numpy(sig_h).to(DEV)
    _, saved = ssw.gated_sa_swa_forward_train(q, k, v, sig, w, causal, g)
    ref = ssw.gated_sa_swa_backward(q, k, v, sig, w, causal, g, saved, dy)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg = torch.empty((2, B, n, Hq), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    got = ssw.gated_sa_swa_backward_noalloc(q, k, v, sig, w, causal, g, saved, dy, dq, dk, dv, dg)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    for name, a, b in zip(("dq", "dk", "dv", "dgates"), ref, got):
        assert torch.equal(a, b), name


def test_noalloc_backward_equals_backward_on_two_calls_second_smaller():
    _case(9100, 2, 2048, 8, 2, 128, 128, True)
    _case(9101, 1, 700, 4, 2, 64, 33, False)
