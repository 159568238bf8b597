"""GPU parity of the decode step (one new token per batch row over a KV cache) against the fp64
oracle, through the C ABI.

Reading R20: decoding position t is row t of causal SA over the full context n_max with one sigma
per layer.  Caches and queries are seeded N(0, 1), gates sigmoid(N(0, 1)), sigma from the seeded
generator (asserted equal on both sides); positions per batch row differ and include 0, small
t < w and n_max - 1.  Bars: fp32 1e-5, bf16 the forward bar (test_gpu_parity.py).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import stochastic_sliding_window_amd as ssw
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _tol(ref, dt):
    if dt == "f32":
        return np.full(ref.shape, 1e-5)
    mag = np.maximum(np.abs(ref), 1e-30)
    half_spacing = np.exp2(np.floor(np.log2(mag)) - 8.0)
    return 1.5e-2 + np.maximum(0.0, half_spacing - 2.0 ** -7)


def _check(got, ref, dt, what):
    err = np.abs(_np(got) - ref)
    bad = err > _tol(ref, dt)
    assert not bad.any(), f"{what}: {int(bad.sum())} over the bar, max err {err.max():.3e}"
    return float(err.max())


def _setup(seed, B, n, Hq, Hkv, d, dt, positions):
    q_all, k, v = synth.qkv(seed, B, n, Hq, Hkv, d, dt)
    pos = np.asarray(positions, dtype=np.int32)
    q = q_all[torch.arange(B), torch.from_numpy(pos).long()].contiguous()   # [B, Hq, d]
    g = synth.gates(seed, B, 1, Hq)[:, :, 0].contiguous()                   # [2, B, Hq]
    sig_np, inv_np = ssw.make_permutation(seed + 1, n, with_inverse=True)
    np.testing.assert_array_equal(sig_np, oracle.make_permutation(seed + 1, n))
    dev = dict(q=q.to(DEV), k=k.to(DEV), v=v.to(DEV), g=g.to(DEV),
               sigma=torch.from_numpy(sig_np).to(DEV), inv=torch.from_numpy(inv_np).to(DEV),
               pos=torch.from_numpy(pos).to(DEV))
    host = dict(q=q, k=k, v=v, g=g, sigma=sig_np, pos=pos, q_all=q_all)
    return host, dev


SHAPES = [  # (B, n_max, Hq, Hkv, d)
    (5, 300, 8, 2, 128),
    (3, 1000, 8, 1, 64),
    (4, 200, 4, 4, 128),
]


def _positions(B, n, w, seed):
    r = np.random.default_rng(seed)
    base = [0, min(n - 1, max(1, w - 1)), n - 1]
    return (base + r.integers(0, n, size=B).tolist())[:B]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("w", [1, 16, 130, 100000])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}n{}h{}x{}d{}".format(*s))
def test_decode_matches_oracle(shape, w, dt):
    B, n, Hq, Hkv, d = shape
    seed = 900 + n + Hq + d
    host, dev = _setup(seed, B, n, Hq, Hkv, d, dt, _positions(B, n, min(w, n), seed))
    q, k, v, pos = host["q"], host["k"], host["v"], host["pos"]
    errs = []
    y = ssw.sa_decode(dev["q"], dev["k"], dev["v"], dev["sigma"], dev["inv"], dev["pos"], w)
    errs.append(_check(y, oracle.sa_decode(q, k, v, host["sigma"], w, pos), dt, "sa"))
    y = ssw.swa_decode(dev["q"], dev["k"], dev["v"], dev["pos"], w, gate=dev["g"][1].contiguous())
    errs.append(_check(y, oracle.swa_decode(q, k, v, w, pos, host["g"][1]), dt, "swa gated"))
    y = ssw.gated_sa_swa_decode(dev["q"], dev["k"], dev["v"], dev["sigma"], dev["inv"], dev["pos"],
                                w, dev["g"])
    errs.append(_check(y, oracle.gated_decode(q, k, v, host["sigma"], w, pos, host["g"]), dt,
                       "gated"))
    torch.cuda.synchronize()
    _say(f"decode {shape} w={w} {dt}: sa/swa/gated max err {errs}")


def test_decode_equals_forward_rows_on_gpu():
    """Decoding every position of a sequence gives the forward kernel's rows (both on the GPU)."""
    B, n, Hq, Hkv, d, w = 1, 160, 8, 2, 128, 24
    q_all, k, v = synth.qkv(77, B, n, Hq, Hkv, d, "bf16")
    sig_np, inv_np = ssw.make_permutation(78, n, with_inverse=True)
    sigma, inv = torch.from_numpy(sig_np).to(DEV), torch.from_numpy(inv_np).to(DEV)
    qd, kd, vd = q_all.to(DEV), k.to(DEV), v.to(DEV)
    fwd = _np(ssw.sa_forward(qd, kd, vd, sigma, w, True))
    # every position as its own batch row over the same cache
    kb = kd.expand(n, -1, -1, -1).contiguous()
    vb = vd.expand(n, -1, -1, -1).contiguous()
    pos = torch.arange(n, dtype=torch.int32, device=DEV)
    dec = _np(ssw.sa_decode(qd[0].contiguous(), kb, vb, sigma, inv, pos, w))
    assert np.abs(dec - fwd[0]).max() <= 2 * 2.0 ** -8 * max(1.0, float(np.abs(fwd).max()))


def test_out_of_range_position_gives_nan_row_only():
    B, n, Hq, Hkv, d = 3, 64, 4, 2, 64
    host, dev = _setup(5, B, n, Hq, Hkv, d, "bf16", [3, 10, 20])
    dev["pos"][1] = n  # out of range
    y = _np(ssw.gated_sa_swa_decode(dev["q"], dev["k"], dev["v"], dev["sigma"], dev["inv"],
                                    dev["pos"], 8, dev["g"]))
    assert np.isnan(y[1]).all() and np.isfinite(y[[0, 2]]).all()


def test_uninitialised_cache_past_t_is_never_read():
    B, n, Hq, Hkv, d, w = 2, 128, 4, 1, 128, 40
    host, dev = _setup(6, B, n, Hq, Hkv, d, "bf16", [50, 90])
    for b, t in enumerate(host["pos"]):
        dev["k"][b, t + 1:] = float("nan")
        dev["v"][b, t + 1:] = float("nan")
    y = ssw.gated_sa_swa_decode(dev["q"], dev["k"], dev["v"], dev["sigma"], dev["inv"],
                                dev["pos"], w, dev["g"])
    ref = oracle.gated_decode(host["q"], host["k"], host["v"], host["sigma"], w, host["pos"],
                              host["g"])
    _check(y, ref, "bf16", "nan-padded cache")


def test_long_context_decode_batch():
    """The bench's shape: Qwen3-8B-shaped heads (32 / 8, d 128), n_max 32768, w 128, bf16."""
    B, n, Hq, Hkv, d, w = 16, 32768, 32, 8, 128, 128
    r = np.random.default_rng(11)
    positions = [0, 127, 32767] + r.integers(0, n, size=B - 3).tolist()
    host, dev = _setup(12, B, n, Hq, Hkv, d, "bf16", positions)
    y = ssw.gated_sa_swa_decode(dev["q"], dev["k"], dev["v"], dev["sigma"], dev["inv"],
                                dev["pos"], w, dev["g"])
    ref = oracle.gated_decode(host["q"], host["k"], host["v"], host["sigma"], w, host["pos"],
                              host["g"])
    _say(f"long-context decode max err {_check(y, ref, 'bf16', 'long'):.3e}")
