"""GPU parity of the training path (forward with log-sum-exp, backward, gated forward/backward)
against the fp64 CPU oracle, through the C ABI.

Inputs are bf16 (the backward takes bf16 only): Q, K, V and the upstream gradient dY ~ N(0, 1),
gates sigmoid(N(0, 1)), sigma from the seeded generator on each side (asserted equal).  The
oracle computes the exact gradients of the exact forward on the same bf16 values.

Bars:
  * forward outputs: the forward bar (1.5e-2 on unit-variance outputs, see test_gpu_parity.py);
    the stored y_sa / y_swa equal the inference kernels' outputs bit for bit;
  * lse: 5e-3 absolute.  The kernel's row sum adds the bf16-rounded weights that enter the P*V
    product (relative error <= 2^-8, bf16's unit roundoff, each; so <= 2^-8 for the sum and
    <= 2^-8 = 3.9e-3 for its log), plus fp32 rounding of the scores, exp2 and log2;
  * gradients: max |gpu - oracle| <= 1.5e-2 * max |oracle| per tensor -- the forward's bar,
    which is stated for unit-scale outputs, applied to each gradient at its own scale.  The
    error sources are the bf16 roundings of P and dS before the gradient products, of A in
    Delta, and of the stored result (relative 2^-8 each, bf16's unit roundoff); the bar is
    about four of them.
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
GRAD_BAR = 1.5e-2
LSE_BAR = 5e-3


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _sigma(seed, n):
    prod = ssw.make_permutation(seed, n)
    ref = oracle.make_permutation(seed, n)
    np.testing.assert_array_equal(prod, ref)
    return torch.from_numpy(prod).to(DEV), ref


def _inputs(seed, B, n, Hq, Hkv, d):
    q, k, v = synth.qkv(seed, B, n, Hq, Hkv, d, "bf16")
    g = synth.gates(seed, B, n, Hq)
    dy = synth.upstream_grad(seed, B, n, Hq, d, "bf16")
    host = (q, k, v, g, dy)
    return host, tuple(t.to(DEV) for t in host)


def _grad_err(name, gpu, ref):
    """max |gpu - ref| / max |ref|, asserted <= GRAD_BAR."""
    got = _np(gpu) if hasattr(gpu, "detach") else gpu
    scale = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    rel = err / scale if scale > 0 else err
    if rel > GRAD_BAR:
        i = np.unravel_index(np.argmax(np.abs(got - ref)), ref.shape)
        raise AssertionError(f"{name}: max err {err:.4e} = {rel:.4e} x max|ref| {scale:.4e}; "
                             f"worst at {i}: got {got[i]}, oracle {ref[i]}")
    return rel


def _fwd_tol(ref):
    mag = np.maximum(np.abs(ref), 1e-30)
    half_spacing = np.exp2(np.floor(np.log2(mag)) - 8.0)
    return 1.5e-2 + np.maximum(0.0, half_spacing - 2.0 ** -7)


# (B, n, Hq, Hkv, d, w): several workgroup tiles and ragged tails; GQA group sizes 1, 2, 3, 4, 8, 32
SHAPES = [
    (1, 300, 8, 2, 128, 16),
    (2, 517, 4, 4, 64, 40),
    (1, 200, 12, 4, 128, 7),
    (1, 389, 8, 2, 64, 33),
    (1, 130, 8, 1, 128, 130),   # window covers the sequence
    (1, 300, 32, 1, 64, 24),    # G = 32: a query-column tile is 4 slots
]


def _ids(s):
    return "B{}n{}h{}x{}d{}w{}".format(*s)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("path", ["sa", "swa"])
@pytest.mark.parametrize("shape", SHAPES, ids=_ids)
def test_backward_matches_oracle(shape, path, causal, gated):
    B, n, Hq, Hkv, d, w = shape
    seed = 7000 + 13 * n + Hq
    host, (q, k, v, g, dy) = _inputs(seed, B, n, Hq, Hkv, d)
    gate = g[0].contiguous() if gated else None
    if path == "sa":
        sig_dev, sig = _sigma(seed + 1, n)
        out, lse = ssw.sa_forward_lse(q, k, v, sig_dev, w, causal)
        dq, dk, dv, dg = ssw.sa_backward(q, k, v, sig_dev, w, causal, out, lse, dy, gate=gate)
    else:
        sig = None
        out, lse = ssw.swa_forward_lse(q, k, v, w, causal)
        dq, dk, dv, dg = ssw.swa_backward(q, k, v, w, causal, out, lse, dy, gate=gate)
    torch.cuda.synchronize()
    qh, kh, vh, gh, dyh = host
    gate_h = gh[0].double().numpy() if gated else None
    rdq, rdk, rdv, rdg = oracle.attention_backward(qh, kh, vh, sig, w, causal, dyh.double(), gate_h)
    rlse = oracle.attention_lse_rows(qh, kh, sig, w, causal)
    lse_err = float(np.abs(_np(lse) - rlse).max())
    assert lse_err <= LSE_BAR, lse_err
    errs = [_grad_err(nm, a, r) for nm, a, r in
            (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv), ("dgate", dg, rdg))]
    _say(f"{_ids(shape)} {path} causal={causal} gated={gated}: lse {lse_err:.2e}, "
         f"dq/dk/dv/dg rel {errs[0]:.2e}/{errs[1]:.2e}/{errs[2]:.2e}/{errs[3]:.2e}")


# Larger grids (256 and more workgroups per kernel, several per CU in flight) with ragged last
# tiles (1100 = 8 * 128 + 76, 800 = 6 * 128 + 32), d = 64 and d = 128
LARGER = [
    ((4, 1100, 16, 16, 64, 40), "sa", True, False),
    ((4, 1100, 16, 16, 64, 40), "sa", False, True),
    ((4, 1100, 16, 16, 64, 40), "swa", True, True),
    ((2, 800, 64, 32, 128, 30), "sa", True, True),
    ((2, 800, 64, 32, 128, 30), "swa", False, False),
    # the dK/dV kernel keeps a table of its chunk columns' rows when a workgroup has at most 56
    # chunks and reads sigma segments otherwise; at n 1600, G 4 the workgroups have up to 56
    # chunks (w 161), 56 and 64 in one launch (w 190), and 57 and more past the table (w 194)
    ((1, 1600, 8, 2, 128, 161), "sa", True, True),
    ((1, 1600, 8, 2, 128, 190), "sa", True, False),
    ((1, 1600, 8, 2, 128, 194), "sa", False, True),
    ((1, 1600, 8, 2, 128, 194), "swa", False, False),
    ((1, 1600, 8, 2, 64, 194), "sa", True, True),    # the same at d 64
]


@pytest.mark.parametrize("shape,path,causal,gated", LARGER,
                         ids=lambda c: _ids(c) if isinstance(c, tuple) else str(c))
def test_backward_larger_grids(shape, path, causal, gated):
    """Every gradient of every row against the oracle on grids of hundreds of workgroups."""
    test_backward_matches_oracle(shape, path, causal, gated)


def test_forward_lse_output_equals_inference_forward():
    B, n, Hq, Hkv, d, w = 1, 700, 8, 2, 128, 64
    host, (q, k, v, g, dy) = _inputs(11, B, n, Hq, Hkv, d)
    sig_dev, _ = _sigma(12, n)
    for causal in (True, False):
        out, _ = ssw.sa_forward_lse(q, k, v, sig_dev, w, causal)
        assert torch.equal(out, ssw.sa_forward(q, k, v, sig_dev, w, causal))
        out, _ = ssw.swa_forward_lse(q, k, v, w, causal)
        assert torch.equal(out, ssw.swa_forward(q, k, v, w, causal))


def test_accumulate_adds_to_given_gradients():
    B, n, Hq, Hkv, d, w = 1, 260, 8, 2, 64, 24
    host, (q, k, v, g, dy) = _inputs(21, B, n, Hq, Hkv, d)
    sig_dev, _ = _sigma(22, n)
    out, lse = ssw.sa_forward_lse(q, k, v, sig_dev, w, True)
    dq0, dk0, dv0, _ = ssw.sa_backward(q, k, v, sig_dev, w, True, out, lse, dy)
    base = [torch.randn(t.shape, generator=torch.Generator().manual_seed(23 + i)).to(t.dtype).to(DEV)
            for i, t in enumerate((dq0, dk0, dv0))]
    acc = [b.clone() for b in base]
    ssw.sa_backward(q, k, v, sig_dev, w, True, out, lse, dy, dq=acc[0], dk=acc[1], dv=acc[2],
                    accumulate=True, want_dgate=False)
    torch.cuda.synchronize()
    for a, b0, gr in zip(acc, base, (dq0, dk0, dv0)):
        ref = _np(b0) + _np(gr)
        # one extra bf16 rounding of the sum and the first result's own rounding
        assert float(np.abs(_np(a) - ref).max()) <= 2.0 ** -7 * max(1.0, float(np.abs(ref).max()))


@pytest.mark.parametrize("shape", [(1, 1, 4, 2, 64, 8), (1, 31, 4, 1, 128, 1), (2, 33, 2, 2, 64, 5)],
                         ids=_ids)
def test_backward_edge_sizes(shape):
    """One token, a window of one (gradients of q and k vanish), a chunk plus one."""
    B, n, Hq, Hkv, d, w = shape
    host, (q, k, v, g, dy) = _inputs(31 + n, B, n, Hq, Hkv, d)
    sig_dev, sig = _sigma(32 + n, n)
    out, lse = ssw.sa_forward_lse(q, k, v, sig_dev, w, True)
    dq, dk, dv, dg = ssw.sa_backward(q, k, v, sig_dev, w, True, out, lse, dy, gate=g[0].contiguous())
    torch.cuda.synchronize()
    qh, kh, vh, gh, dyh = host
    rdq, rdk, rdv, rdg = oracle.attention_backward(qh, kh, vh, sig, w, True, dyh.double(),
                                                   gh[0].double().numpy())
    for nm, a, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv), ("dgate", dg, rdg)):
        if np.abs(r).max() == 0:
            # w = 1: every row attends to itself alone, so the score gradients are exactly zero;
            # the kernel's dP - Delta is a difference of two fp32 sums of the same products
            assert float(np.abs(_np(a)).max()) <= 1e-3, nm
        else:
            _grad_err(nm, a, r)


def test_empty_backward_is_noop():
    z = torch.zeros(1, 0, 4, 64, dtype=torch.bfloat16, device=DEV)
    zk = torch.zeros(1, 0, 2, 64, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 0, 4, dtype=torch.float32, device=DEV)
    ssw.swa_backward(z, zk, zk, 8, True, z, lse, z)


@pytest.mark.parametrize("causal", [True, False])
def test_gated_training_forward_and_backward(causal):
    B, n, Hq, Hkv, d, w = 1, 333, 8, 2, 128, 20
    host, (q, k, v, g, dy) = _inputs(41, B, n, Hq, Hkv, d)
    sig_dev, sig = _sigma(42, n)
    out, saved = ssw.gated_sa_swa_forward_train(q, k, v, sig_dev, w, causal, g)
    y_sa, lse_sa, y_swa, lse_swa = saved
    assert torch.equal(y_sa, ssw.sa_forward(q, k, v, sig_dev, w, causal))
    assert torch.equal(y_swa, ssw.swa_forward(q, k, v, w, causal))
    dq, dk, dv, dgates = ssw.gated_sa_swa_backward(q, k, v, sig_dev, w, causal, g, saved, dy)
    torch.cuda.synchronize()
    qh, kh, vh, gh, dyh = host
    ref = oracle.gated_forward(qh, kh, vh, sig, w, causal, gh)
    err = np.abs(_np(out) - ref)
    assert (err <= _fwd_tol(ref)).all(), float(err.max())
    rdq, rdk, rdv, rdg = oracle.gated_backward(qh, kh, vh, sig, w, causal, gh, dyh.double())
    errs = [_grad_err(nm, a, r) for nm, a, r in
            (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv), ("dgates", dgates, rdg))]
    _say(f"gated causal={causal}: fwd {float(err.max()):.2e}, rel {errs}")


def test_gated_backward_full_size_sampled_rows():
    """The long-context layer (B1 n32768 Hq32 Hkv8 d128 causal w128), as the backward bench runs
    it: dq and dgates of sampled query rows, dk and dv of sampled key rows, against the oracle's
    sampled-row gradients."""
    wl = synth.workload(4)
    B, n, Hq, Hkv, d, w = wl.B, wl.n, wl.Hq, wl.Hkv, wl.d, 128
    seed = synth.data_seed(4, 0)
    host, (q, k, v, g, dy) = _inputs(seed, B, n, Hq, Hkv, d)
    sig_dev, sig = _sigma(synth.sigma_seed(4, 0), n)
    _say("full-size gated training forward + backward on the GPU")
    out, saved = ssw.gated_sa_swa_forward_train(q, k, v, sig_dev, w, True, g)
    dq, dk, dv, dgates = ssw.gated_sa_swa_backward(q, k, v, sig_dev, w, True, g, saved, dy)
    torch.cuda.synchronize()
    qh, kh, vh, gh, dyh = host
    r = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, n - 1], r.choice(n, 7, replace=False)]))
    keys = np.unique(np.concatenate([[0, n - 1], r.choice(n, 3, replace=False)]))
    dyd = dyh.double()
    g_sa, g_swa = gh[0].double().numpy(), gh[1].double().numpy()
    _say(f"oracle on {len(rows)} query rows and {len(keys)} key rows")
    q1, dg1 = oracle.attention_backward_query_rows(qh, kh, vh, sig, w, True, dyd, g_sa, rows)
    q2, dg2 = oracle.attention_backward_query_rows(qh, kh, vh, None, w, True, dyd, g_swa, rows)
    k1, v1 = oracle.attention_backward_key_rows(qh, kh, vh, sig, w, True, dyd, g_sa, keys)
    k2, v2 = oracle.attention_backward_key_rows(qh, kh, vh, None, w, True, dyd, g_swa, keys)
    errs = [_grad_err("dq rows", _np(dq)[:, rows], q1 + q2),
            _grad_err("dg_sa rows", _np(dgates[0])[:, rows], dg1),
            _grad_err("dg_swa rows", _np(dgates[1])[:, rows], dg2),
            _grad_err("dk rows", _np(dk)[:, keys], k1 + k2),
            _grad_err("dv rows", _np(dv)[:, keys], v1 + v2)]
    _say(f"full-size sampled rel errors {['%.2e' % e for e in errs]}")
