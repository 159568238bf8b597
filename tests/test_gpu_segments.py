"""GPU parity where a workgroup's band is longer than the sigma segment its kernel holds in LDS.

The forward kernels hold sigma for up to 2048 band keys at a time (1024 in the three-waves
builds); the backward kernels hold 2048 slots.  A band longer than that makes a workgroup reload
sigma part way through its loop (and, in the gated layer's SA pass, fetch its intermediate rows
during the last chunk of the last segment).  With G = 4 query heads per KV head a forward tile
spans 33 slots, so its band is 33 + 2 (w - 1) keys: w = 1100 gives 2231 keys, two segments, for
all but the tiles near the sequence ends.  [SA-ja] 中核メカニズム step 2 allows any window w.

Rows compared: the first and last original rows, the tokens at the slots around tile and segment
boundaries, and random rows; bars as in test_gpu_parity.py (bf16 1.5e-2, fp32 1e-5) and
test_gpu_backward.py (gradients 1.5e-2 x max |oracle| per tensor).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import stochastic_sliding_window_amd as ssw
import synth

from test_gpu_parity import _maxerr

pytestmark = pytest.mark.gpu

DEV = "cuda"
W_LONG = 1100


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _sigma(seed, n):
    prod = ssw.make_permutation(seed, n)
    ref = oracle.make_permutation(seed, n)
    np.testing.assert_array_equal(prod, ref)
    return torch.from_numpy(prod).to(DEV), ref


def _rows(sig, n, seed, count=24):
    """Original rows: ends, tokens at slots around tile (32k) and segment (2048) boundaries, and
    random rows."""
    r = np.random.default_rng(seed)
    slots = [0, 1, 31, 32, 33, 1024, 2047, 2048, 2049, n - 33, n - 2, n - 1]
    rows = {0, n - 1} | {int(sig[s]) for s in slots if 0 <= s < n}
    rows |= set(r.choice(n, size=count, replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("path", ["sa", "gated"])
def test_forward_band_over_two_sigma_segments_bf16(path, causal):
    B, n, Hq, Hkv, d, w = 1, 4096, 8, 2, 128, W_LONG
    seed = 8100 + (1 if causal else 0)
    q, k, v = synth.qkv(seed, B, n, Hq, Hkv, d, "bf16")
    g = synth.gates(seed, B, n, Hq)
    sig_dev, sig = _sigma(seed + 1, n)
    qd, kd, vd, gd = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV)
    _say(f"segments {path} causal={causal} n={n} w={w} bf16")
    if path == "sa":
        out = ssw.sa_forward(qd, kd, vd, sig_dev, w, causal)
    else:
        out = ssw.gated_sa_swa_forward(qd, kd, vd, sig_dev, w, causal, gd)
    torch.cuda.synchronize()
    rows = _rows(sig, n, seed)
    if path == "sa":
        ref = oracle.sa_rows(q, k, v, sig, w, causal, rows)
    else:
        ref = oracle.gated_forward(q, k, v, sig, w, causal, g, rows)
    err = _maxerr(out[:, rows], ref, "bf16")
    _say(f"   {len(rows)} rows, max err {err:.3e}")


@pytest.mark.parametrize("path", ["sa", "gated"])
def test_forward_band_over_two_sigma_segments_fp32(path):
    B, n, Hq, Hkv, d, w = 1, 4096, 4, 1, 64, W_LONG
    seed = 8200
    q, k, v = synth.qkv(seed, B, n, Hq, Hkv, d, "f32")
    g = synth.gates(seed, B, n, Hq)
    sig_dev, sig = _sigma(seed + 1, n)
    qd, kd, vd, gd = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV)
    _say(f"segments {path} causal n={n} w={w} fp32")
    if path == "sa":
        out = ssw.sa_forward(qd, kd, vd, sig_dev, w, True)
    else:
        out = ssw.gated_sa_swa_forward(qd, kd, vd, sig_dev, w, True, gd)
    torch.cuda.synchronize()
    rows = _rows(sig, n, seed)
    if path == "sa":
        ref = oracle.sa_rows(q, k, v, sig, w, True, rows)
    else:
        ref = oracle.gated_forward(q, k, v, sig, w, True, g, rows)
    err = _maxerr(out[:, rows], ref, "f32")
    _say(f"   {len(rows)} rows, max err {err:.3e}")


def _keys(sig, n, seed, count=3):
    """Key rows for dk/dv: late tokens (original index in the last 60, so that few queries attend
    to them and the oracle's per-key sum stays cheap) whose slots lie in the middle of the
    sequence, where a dK/dV tile's band of query slots spans two sigma segments."""
    inv = oracle.inverse_permutation(sig)
    cand = [j for j in range(n - 60, n) if 1200 <= inv[j] <= n - 1200]
    r = np.random.default_rng(seed)
    return np.array(sorted(r.choice(cand, size=min(count, len(cand)), replace=False).tolist()))


def _grad_err(name, got, ref):
    scale = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    rel = err / scale if scale > 0 else err
    assert rel <= 1.5e-2, f"{name}: max err {err:.4e} = {rel:.4e} x max|ref| {scale:.4e}"
    return rel


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("causal,B,d", [(True, 1, 128), (False, 1, 128), (True, 8, 128),
                                         (True, 1, 64)])
def test_sa_backward_band_over_two_sigma_segments(causal, B, d):
    """dq of sampled query rows and (causal) dk, dv of sampled key rows of SA with a gate, at a
    band over two sigma segments of the dQ (2231 keys per tile) and dK/dV (128 + 2198 query
    slots per tile) kernels; B = 8 also checks batch rows past the first, d = 64 the other
    head size's build of both kernels."""
    n, Hq, Hkv, w = 4096, 8, 2, W_LONG
    seed = 8300 + (1 if causal else 0) + (2 if d == 64 else 0)
    q, k, v = synth.qkv(seed, B, n, Hq, Hkv, d, "bf16")
    g = synth.gates(seed, B, n, Hq)
    dy = synth.upstream_grad(seed, B, n, Hq, d, "bf16")
    sig_dev, sig = _sigma(seed + 1, n)
    qd, kd, vd, dyd = q.to(DEV), k.to(DEV), v.to(DEV), dy.to(DEV)
    gate = g[0].contiguous().to(DEV)
    _say(f"segments sa backward causal={causal} B={B} d={d} n={n} w={w}")
    out, lse = ssw.sa_forward_lse(qd, kd, vd, sig_dev, w, causal)
    dq, dk, dv, dg = ssw.sa_backward(qd, kd, vd, sig_dev, w, causal, out, lse, dyd, gate=gate)
    torch.cuda.synchronize()
    rows = _rows(sig, n, seed, count=10)
    gh = g[0].double().numpy()
    rq, rdg = oracle.attention_backward_query_rows(q, k, v, sig, w, causal, dy.double(), gh, rows)
    errs = [_grad_err("dq", _np(dq)[:, rows], rq), _grad_err("dgate", _np(dg)[:, rows], rdg)]
    if causal:
        # non-causal: every query of a key's band attends to it, about 2w of them, each with a
        # neighbour set of about 2w keys, which puts the oracle's per-key sum at about a minute
        # per key; the dK/dV kernel's segment reload is the same code in both modes
        keys = _keys(sig, n, seed + 7)
        rk, rv = oracle.attention_backward_key_rows(q, k, v, sig, w, causal, dy.double(), gh, keys)
        errs += [_grad_err("dk", _np(dk)[:, keys], rk), _grad_err("dv", _np(dv)[:, keys], rv)]
    _say(f"   rel errors {['%.2e' % e for e in errs]}")


def test_gated_backward_band_over_two_sigma_segments():
    B, n, Hq, Hkv, d, w = 1, 4096, 8, 2, 128, W_LONG
    seed = 8400
    q, k, v = synth.qkv(seed, B, n, Hq, Hkv, d, "bf16")
    g = synth.gates(seed, B, n, Hq)
    dy = synth.upstream_grad(seed, B, n, Hq, d, "bf16")
    sig_dev, sig = _sigma(seed + 1, n)
    qd, kd, vd, gd, dyd = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), dy.to(DEV)
    _say(f"segments gated backward causal n={n} w={w}")
    out, saved = ssw.gated_sa_swa_forward_train(qd, kd, vd, sig_dev, w, True, gd)
    dq, dk, dv, dgates = ssw.gated_sa_swa_backward(qd, kd, vd, sig_dev, w, True, gd, saved, dyd)
    torch.cuda.synchronize()
    rows = _rows(sig, n, seed, count=8)
    keys = _keys(sig, n, seed + 7)
    dyh = dy.double()
    g_sa, g_swa = g[0].double().numpy(), g[1].double().numpy()
    q1, dg1 = oracle.attention_backward_query_rows(q, k, v, sig, w, True, dyh, g_sa, rows)
    q2, dg2 = oracle.attention_backward_query_rows(q, k, v, None, w, True, dyh, g_swa, rows)
    k1, v1 = oracle.attention_backward_key_rows(q, k, v, sig, w, True, dyh, g_sa, keys)
    k2, v2 = oracle.attention_backward_key_rows(q, k, v, None, w, True, dyh, g_swa, keys)
    errs = [_grad_err("dq", _np(dq)[:, rows], q1 + q2),
            _grad_err("dg_sa", _np(dgates[0])[:, rows], dg1),
            _grad_err("dg_swa", _np(dgates[1])[:, rows], dg2),
            _grad_err("dk", _np(dk)[:, keys], k1 + k2), _grad_err("dv", _np(dv)[:, keys], v1 + v2)]
    _say(f"   rel errors {['%.2e' % e for e in errs]}")
