"""GPU parity of the per-batch / per-KV-head sigma variant against the fp64 oracle.

Each (batch row b, KV head g) runs SA with its own permutation sigma_bg; the oracle result is the
pinned single-sigma SA applied to that (b, g) slice (its G query heads and one KV head) with
sigma_bg.  Bars as in test_gpu_parity.py (fp32 1e-5, bf16 1.5e-2 with the |Y| >= 4 allowance).
"""

import numpy as np
import pytest
import torch

import oracle
import stochastic_sliding_window_amd as ssw
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _tol(ref, dt):
    if dt == "f32":
        return np.full(ref.shape, 1e-5)
    mag = np.maximum(np.abs(ref), 1e-30)
    return 1.5e-2 + np.maximum(0.0, np.exp2(np.floor(np.log2(mag)) - 8.0) - 2.0 ** -7)


def _sigmas(kind, B, Hkv, n, seed):
    shape = {"batch": (B,), "head": (Hkv,), "both": (B, Hkv)}[kind]
    flat = [ssw.make_permutation(seed + i, n) for i in range(int(np.prod(shape)))]
    for i, s in enumerate(flat):
        np.testing.assert_array_equal(s, oracle.make_permutation(seed + i, n))
    return np.stack(flat).reshape(*shape, n)


def _sigma_of(sig, kind, b, g):
    return {"batch": lambda: sig[b], "head": lambda: sig[g], "both": lambda: sig[b, g]}[kind]()


def _oracle(host, sig, kind, w, causal, gated):
    q, k, v, gates = host
    B, n, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    out = np.empty((B, n, Hq, d))
    for b in range(B):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            qs, ks, vs = q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1]
            y = oracle.sa_rows(qs, ks, vs, _sigma_of(sig, kind, b, g), w, causal)
            if gated:
                gs = gates[:, b:b + 1, :, hs].double().numpy()
                y = gs[0][..., None] * y + gs[1][..., None] * oracle.swa_rows(qs, ks, vs, w, causal)
            out[b:b + 1, :, hs] = y
    return out


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("kind", ["batch", "head", "both"])
@pytest.mark.parametrize("dt,shape", [("bf16", (3, 300, 8, 2, 128, 20)),
                                      ("f32", (2, 150, 4, 4, 64, 9))])
def test_per_row_and_head_sigma(kind, gated, dt, shape):
    B, n, Hq, Hkv, d, w = shape
    seed = 600 + n
    q, k, v = synth.qkv(seed, B, n, Hq, Hkv, d, dt)
    g = synth.gates(seed, B, n, Hq)
    sig = _sigmas(kind, B, Hkv, n, seed)
    dq, dk, dv, dg = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV)
    ds = torch.from_numpy(sig).to(DEV).contiguous()
    for causal in (True, False):
        if gated:
            y = ssw.gated_sa_swa_forward_ex(dq, dk, dv, ds, w, causal, dg)
        else:
            y = ssw.sa_forward_ex(dq, dk, dv, ds, w, causal)
        torch.cuda.synchronize()
        ref = _oracle((q, k, v, g), sig, kind, w, causal, gated)
        err = np.abs(_np(y) - ref)
        assert (err <= _tol(ref, dt)).all(), float(err.max())


def test_shared_sigma_strides_equal_the_plain_call():
    B, n, Hq, Hkv, d, w = 2, 257, 8, 2, 128, 33
    q, k, v = (t.to(DEV) for t in synth.qkv(5, B, n, Hq, Hkv, d, "bf16"))
    g = synth.gates(5, B, n, Hq).to(DEV)
    s = torch.from_numpy(ssw.make_permutation(6, n)).to(DEV)
    assert torch.equal(ssw.sa_forward_ex(q, k, v, s, w, True), ssw.sa_forward(q, k, v, s, w, True))
    # the same permutation repeated per (row, head) gives the shared-sigma result too
    rep = s.expand(B, Hkv, n).contiguous()
    assert torch.equal(ssw.gated_sa_swa_forward_ex(q, k, v, rep, w, True, g),
                       ssw.gated_sa_swa_forward(q, k, v, s, w, True, g))
