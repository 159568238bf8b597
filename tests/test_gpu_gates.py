"""GPU parity of the gate projections (ssw_gate_projection) against the fp64 oracle.

x ~ N(0, 1), w ~ N(0, 1/Hm) (so each logit is ~ N(0, 1)), bias ~ N(0, 1), bf16 x and w as given
to both sides.  Bar 2e-5 on the gates: the kernel accumulates the Hm products in fp32 (error of
order sqrt(Hm) * 2^-24 on a unit logit, about 4e-6 at Hm = 4096) and its sigmoid uses the fast
exp (relative error about 1e-6); the sigmoid's slope is at most 1/4.
"""

import numpy as np
import pytest
import torch

import oracle
import stochastic_sliding_window_amd as ssw
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"
BAR = 2e-5


@pytest.mark.parametrize("with_bias", [True, False])
@pytest.mark.parametrize("B,n,Hm,Hq", [(2, 500, 4096, 32), (1, 130, 64, 1), (1, 300, 2048, 16),
                                       (1, 257, 1024, 48), (3, 7, 16, 64)])
def test_gate_projection_matches_oracle(B, n, Hm, Hq, with_bias):
    x, w_t, bias = synth.gate_inputs(B * n + Hm + Hq, B * n, Hm, Hq)
    xd = x.reshape(B, n, Hm).to(DEV)
    g = ssw.gate_projection(xd, w_t.to(DEV), bias.to(DEV) if with_bias else None)
    torch.cuda.synchronize()
    assert tuple(g.shape) == (2, B, n, Hq)
    ref = oracle.gate_projection(x, w_t.double().numpy().T, bias if with_bias else None, B, n, Hq)
    assert np.abs(g.cpu().double().numpy() - ref).max() <= BAR


def test_projected_gates_drive_the_gated_layer():
    """x -> gates on the GPU -> gated forward equals the gated forward with the oracle's gates."""
    B, n, Hq, Hkv, d, Hm, w = 1, 384, 8, 2, 128, 512, 32
    q, k, v = synth.qkv(91, B, n, Hq, Hkv, d, "bf16")
    x, w_t, bias = synth.gate_inputs(92, B * n, Hm, Hq)
    sigma = ssw.make_permutation(93, n)
    dev = [t.to(DEV) for t in (q, k, v)]
    gates = ssw.gate_projection(x.reshape(B, n, Hm).to(DEV), w_t.to(DEV), bias.to(DEV))
    y = ssw.gated_sa_swa_forward(*dev, torch.from_numpy(sigma).to(DEV), w, True, gates)
    torch.cuda.synchronize()
    g_ref = oracle.gate_projection(x, w_t.double().numpy().T, bias, B, n, Hq)
    ref = oracle.gated_forward(q, k, v, sigma, w, True, g_ref)
    assert np.abs(y.float().cpu().numpy() - ref).max() <= 1.5e-2
