"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Every case draws Q, K, V (and gates) from the seeded synthetic generator, runs the library on the
GPU and compares element by element with the oracle on the same values.  sigma is generated on
each side by its own implementation of the published generator and the two are asserted equal
before use.  Bars: fp32 max |err| <= 1e-5; bf16 (fp32 accumulation, unit-variance V) max |err|
<= 1.5e-2; neighbour sets and permutations bit-exact.

The bf16 bar is applied to the bf16 OUTPUT.  Where the exact result has |Y| >= 4 the bf16 grid is
2^-5 wide, so even the correctly rounded value can sit 2^-6 = 0.0156 away from it; there, and only
there, the bar is raised by the excess of that half-spacing over 2^-7 (the half-spacing at the
top of the unit range [2, 4)): tol(Y) = 1.5e-2 + max(0, h(Y) - 2^-7).
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
TOL = {"f32": 1e-5, "bf16": 1.5e-2}


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _sigma(seed, n):
    prod = ssw.make_permutation(seed, n)
    ref = oracle.make_permutation(seed, n)
    np.testing.assert_array_equal(prod, ref)
    return torch.from_numpy(prod).to(DEV), ref


def _data(seed, B, n, Hq, Hkv, d, dt):
    q, k, v = synth.qkv(seed, B, n, Hq, Hkv, d, dt)
    g = synth.gates(seed, B, n, Hq)
    return (q, k, v, g), (q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV))


def _tol(ref, dt):
    """Per-element bar (see the module docstring)."""
    if dt == "f32":
        return np.full(ref.shape, TOL["f32"])
    mag = np.maximum(np.abs(ref), 1e-30)
    half_spacing = np.exp2(np.floor(np.log2(mag)) - 8.0)
    return TOL["bf16"] + np.maximum(0.0, half_spacing - 2.0 ** -7)


def _maxerr(gpu, ref, dt=None):
    """max |gpu - ref|; with dt, also asserts every element is within its bar."""
    got = gpu.detach().float().cpu().numpy().astype(np.float64) if hasattr(gpu, "detach") else gpu
    err = np.abs(got - ref)
    if dt is not None:
        tol = _tol(ref, dt)
        bad = err > tol
        if bad.any():
            i = np.unravel_index(np.argmax(err - tol), err.shape)
            raise AssertionError(f"{int(bad.sum())} elements over the bar; worst at {i}: "
                                 f"got {got[i]}, oracle {ref[i]}, err {err[i]:.4e} > {tol[i]:.4e}")
    return float(err.max())


def _run_path(path, dev, sig_dev, w, causal):
    q, k, v, g = dev
    if path == "sa":
        return ssw.sa_forward(q, k, v, sig_dev, w, causal)
    if path == "sa_gate":
        return ssw.sa_forward(q, k, v, sig_dev, w, causal, gate=g[0].contiguous())
    if path == "swa":
        return ssw.swa_forward(q, k, v, w, causal)
    if path == "gated":
        return ssw.gated_sa_swa_forward(q, k, v, sig_dev, w, causal, g)
    raise ValueError(path)


def _oracle_path(path, host, sig, w, causal, rows=None):
    q, k, v, g = host
    if path == "sa":
        return oracle.sa_rows(q, k, v, sig, w, causal, rows)
    if path == "sa_gate":
        y = oracle.sa_rows(q, k, v, sig, w, causal, rows)
        gg = g[0].double().numpy()
        gg = gg if rows is None else gg[:, rows]
        return gg[..., None] * y
    if path == "swa":
        return oracle.swa_rows(q, k, v, w, causal, rows)
    if path == "gated":
        return oracle.gated_forward(q, k, v, sig, w, causal, g, rows)
    raise ValueError(path)


# --------------------------------------------------------------------------------------------
# The tiny oracle workload: B1 H1 n256 d64 w16 fp32, non-causal and causal, SA / SWA / gated
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("path", ["sa", "swa", "gated", "sa_gate"])
def test_tiny_workload_fp32(path, causal):
    wl = synth.workload(1)
    host, dev = _data(synth.data_seed(1, 0), wl.B, wl.n, wl.Hq, wl.Hkv, wl.d, wl.dtype)
    sig_dev, sig = _sigma(synth.sigma_seed(1, 0), wl.n)
    w = wl.windows[0]
    out = _run_path(path, dev, sig_dev, w, causal)
    torch.cuda.synchronize()
    err = _maxerr(out, _oracle_path(path, host, sig, w, causal), "f32")
    _say(f"tiny {path} causal={causal}: max err {err:.3e}")


# --------------------------------------------------------------------------------------------
# Shapes spanning several workgroup tiles and a ragged tail, GQA group sizes 1, 2, 3, 4, 8
# --------------------------------------------------------------------------------------------

SHAPES = [
    # B, n, Hq, Hkv, d, w
    (2, 1000, 8, 2, 128, 64),
    (1, 777, 4, 4, 64, 40),
    (1, 513, 16, 2, 128, 100),
    (2, 300, 6, 2, 64, 17),
    (1, 2100, 4, 1, 128, 128),
    (1, 300, 16, 1, 128, 33),   # G = 16: a 128-column tile is 8 slots
    (1, 600, 32, 1, 64, 50),    # G = 32: 4 slots per tile
    (1, 200, 64, 1, 64, 20),    # G = 64: 2 slots per tile, a slot's heads split over two waves
]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}n{}Hq{}Hkv{}d{}w{}".format(*s))
def test_parity_shapes(shape, causal, dt):
    B, n, Hq, Hkv, d, w = shape
    seed = 7 * n + w + (1 if causal else 0)
    host, dev = _data(seed, B, n, Hq, Hkv, d, dt)
    sig_dev, sig = _sigma(seed + 99, n)
    for path in ("sa", "swa", "gated"):
        out = _run_path(path, dev, sig_dev, w, causal)
        torch.cuda.synchronize()
        _say(f"{shape} {dt} causal={causal} {path}")
        err = _maxerr(out, _oracle_path(path, host, sig, w, causal), dt)
        _say(f"   max err {err:.3e}")


EDGES = [
    # B, n, Hq, Hkv, d, w
    (1, 1, 2, 1, 64, 4),        # a single token
    (1, 2, 1, 1, 128, 1),       # w = 1: only the token itself
    (3, 31, 4, 2, 64, 8),       # less than one key chunk, three batch rows
    (1, 33, 2, 2, 128, 33),     # w = n: full attention
    (1, 70, 2, 1, 64, 500),     # w > n
    (1, 97, 8, 8, 64, 96),      # w = n - 1
    (1, 257, 1, 1, 64, 1),      # one column past a workgroup tile, w = 1
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("shape", EDGES, ids=lambda s: "B{}n{}Hq{}Hkv{}d{}w{}".format(*s))
def test_parity_edges(shape, causal, dt):
    B, n, Hq, Hkv, d, w = shape
    host, dev = _data(n + w, B, n, Hq, Hkv, d, dt)
    sig_dev, sig = _sigma(n * 3 + 1, n)
    for path in ("sa", "swa", "gated", "sa_gate"):
        out = _run_path(path, dev, sig_dev, w, causal)
        torch.cuda.synchronize()
        _maxerr(out, _oracle_path(path, host, sig, w, causal), dt)


def test_window_covering_sequence_is_full_attention_on_gpu():
    # any sigma, w >= n: SA is plain attention -> compare with torch SDPA on the GPU in fp32
    B, n, Hq, Hkv, d = 1, 200, 4, 2, 64
    host, dev = _data(5, B, n, Hq, Hkv, d, "f32")
    sig_dev, _ = _sigma(6, n)
    q, k, v, _ = dev
    for causal in (False, True):
        out = ssw.sa_forward(q, k, v, sig_dev, n, causal)
        kk = k.repeat_interleave(Hq // Hkv, dim=2)
        vv = v.repeat_interleave(Hq // Hkv, dim=2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q.transpose(1, 2), kk.transpose(1, 2).contiguous(), vv.transpose(1, 2).contiguous(),
            is_causal=causal).transpose(1, 2)
        assert (out - ref).abs().max().item() <= 1e-5


@pytest.mark.parametrize("path", ["swa", "sa"])
def test_full_causal_attention_comparator(path):
    """The full-attention comparator: a window covering the sequence (w = n) on the same kernels.
    At n = 4096 a workgroup's band spans 128 key chunks, i.e. two sigma segments, so this also
    covers the segment reload path.  Sampled rows (first, last, random, a tile boundary) against
    the oracle, bf16 bar."""
    B, n, Hq, Hkv, d = 1, 4096, 8, 2, 128
    w = n
    host, dev = _data(31, B, n, Hq, Hkv, d, "bf16")
    sig_dev, sig = _sigma(32, n)
    q, k, v, _ = dev
    if path == "swa":
        out = ssw.swa_forward(q, k, v, w, True)
    else:
        out = ssw.sa_forward(q, k, v, sig_dev, w, True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 33, n - 2, n - 1],
                                     rng.choice(n, size=40, replace=False)]))
    qh, kh, vh, _ = host
    if path == "swa":
        ref = oracle.swa_rows(qh, kh, vh, w, True, rows)
    else:
        ref = oracle.sa_rows(qh, kh, vh, sig, w, True, rows)
    got = out[:, rows]
    err = _maxerr(got, ref, "bf16")
    _say(f"full causal attention n={n} {path}: max err {err:.3e}")


def test_timed_gated_call_matches_untimed():
    B, n, Hq, Hkv, d, w = 1, 700, 8, 2, 128, 64
    _, dev = _data(21, B, n, Hq, Hkv, d, "bf16")
    sig_dev, _ = _sigma(22, n)
    q, k, v, g = dev
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()
    a = ssw.gated_sa_swa_forward(q, k, v, sig_dev, w, True, g)
    b = ssw.gated_sa_swa_forward(q, k, v, sig_dev, w, True, g, events=evs)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # each pair brackets one kernel (0, 1: the SWA pass; 2, 3: the SA pass); the SA pass runs
    # first, and the SWA pass starts no earlier than it ends
    assert evs[0].elapsed_time(evs[1]) > 0 and evs[2].elapsed_time(evs[3]) > 0
    assert evs[3].elapsed_time(evs[0]) >= 0


def test_empty_inputs_are_noops():
    q = torch.empty(1, 0, 2, 64, device=DEV)
    k = torch.empty(1, 0, 1, 64, device=DEV)
    sig = torch.empty(0, dtype=torch.int32, device=DEV)
    out = ssw.sa_forward(q, k, k, sig, 4, True)
    assert out.shape == q.shape
    q = torch.empty(0, 5, 2, 64, device=DEV)
    k = torch.empty(0, 5, 1, 64, device=DEV)
    sig = torch.arange(5, dtype=torch.int32, device=DEV)
    ssw.gated_sa_swa_forward(q, k, k, sig, 4, True, torch.empty(2, 0, 5, 2, device=DEV))


# --------------------------------------------------------------------------------------------
# Neighbour sets, bit-exact
# --------------------------------------------------------------------------------------------

def _oracle_bits(sig, n, w, causal):
    words = (n + 31) // 32
    bits = np.zeros((n, words), dtype=np.uint32)
    inv = oracle.inverse_permutation(sig) if sig is not None else None
    for i in range(n):
        nb = oracle.sa_neighbours(sig, w, causal, i, inv) if sig is not None else \
            oracle.swa_neighbours(n, w, causal, i)
        for j in nb:
            bits[i, j // 32] |= np.uint32(1 << (int(j) % 32))
    return bits


@pytest.mark.parametrize("n,w", [(1, 1), (37, 5), (256, 16), (100, 300), (64, 1)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mode", ["sa", "swa"])
def test_neighbor_mask_bit_exact(n, w, causal, mode):
    sig_dev, sig = _sigma(1000 + n, n)
    if mode == "swa":
        sig_dev, sig = None, None
    bits = ssw.neighbor_mask(sig_dev, n, w, causal, device=DEV)
    got = bits.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, _oracle_bits(sig, n, w, causal))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_kernel_neighbourhoods_by_probe(causal):
    # Q = 0 makes all in-band scores equal, so row i of the output is the mean of V over N(i).
    # With V one-hot over 64 token indices at a time, Y[i, c] != 0 exactly when token 64t + c is a
    # neighbour of i, and then equals 1/|N(i)|.  This reads the neighbour sets out of the real
    # attention kernel, bit for bit.
    n, w, d = 256, 16, 64
    sig_dev, sig = _sigma(4242, n)
    inv = oracle.inverse_permutation(sig)
    q = torch.zeros(1, n, 1, d, device=DEV)
    k = torch.randn(1, n, 1, d, device=DEV)
    sizes = np.array([len(oracle.sa_neighbours(sig, w, causal, i, inv)) for i in range(n)])
    for t in range(n // d):
        v = torch.zeros(1, n, 1, d, device=DEV)
        v[0, t * d:(t + 1) * d, 0, :] = torch.eye(d, device=DEV)
        y = ssw.sa_forward(q, k, v, sig_dev, w, causal)[0, :, 0, :].cpu().numpy()
        for i in range(n):
            nb = oracle.sa_neighbours(sig, w, causal, i, inv)
            want = np.zeros(d, dtype=bool)
            sel = nb[(nb >= t * d) & (nb < (t + 1) * d)] - t * d
            want[sel] = True
            np.testing.assert_array_equal(y[i] != 0, want, err_msg=f"row {i} block {t}")
            np.testing.assert_allclose(y[i][want], 1.0 / sizes[i], rtol=1e-6)


def test_identity_sigma_matches_swa_kernel():
    B, n, Hq, Hkv, d, w = 1, 600, 8, 2, 128, 64
    _, dev = _data(77, B, n, Hq, Hkv, d, "bf16")
    q, k, v, _ = dev
    ident = torch.arange(n, dtype=torch.int32, device=DEV)
    # Same neighbour sets in both modes.  The two specialisations differ in loop structure (the
    # permuted one consumes two 32-key chunks per step and keeps a lazy running maximum per 64
    # keys; the identity one, sized for three waves per SIMD, one chunk per step; causal SWA also
    # skips the keys right of the query), so they agree up to bf16 rounding, not bit for bit.
    for causal in (False, True):
        a = ssw.sa_forward(q, k, v, ident, w, causal)
        b = ssw.swa_forward(q, k, v, w, causal)
        assert (a.float() - b.float()).abs().max().item() <= 1e-2


# --------------------------------------------------------------------------------------------
# Full-size workloads: sampled rows against the oracle, in the launch configuration of the bench
# --------------------------------------------------------------------------------------------

def _sample_rows(n, count, seed):
    r = np.random.default_rng(seed)
    rows = set(r.choice(n, size=min(count, n), replace=False).tolist())
    rows |= {0, 1, n // 2, n - 2, n - 1}
    return sorted(rows)


@pytest.mark.parametrize("index", [2, 3, 4, 5])
def test_full_size_workloads_sampled_rows(index):
    wl = synth.workload(index)
    host, dev = _data(synth.data_seed(index, 0), wl.B, wl.n, wl.Hq, wl.Hkv, wl.d, wl.dtype)
    layers = sorted({0, wl.layers - 1})
    for layer in layers:
        sig_dev, sig = _sigma(synth.sigma_seed(index, layer), wl.n)
        rows = _sample_rows(wl.n, 24, 31 * index + layer)
        for w in wl.windows:
            for path in wl.paths:
                out = _run_path(path, dev, sig_dev, w, True)
                torch.cuda.synchronize()
                got = out[:, rows].float().cpu().numpy().astype(np.float64)
                ref = _oracle_path(path, host, sig, w, True, rows)
                _say(f"workload {index} layer {layer} w={w} {path} ({len(rows)} rows)")
                err = _maxerr(got, ref, wl.dtype)
                _say(f"   max err {err:.3e}")
                assert torch.isfinite(out).all()


@pytest.mark.parametrize("w", [496, 497])
@pytest.mark.parametrize("causal", [True, False])
def test_sa_alone_build_switch(w, causal):
    """SA alone has two builds: three waves per SIMD when a workgroup's band (ceil(128 / G) + 1
    slots plus 2(w - 1) keys) fits its 1024-entry sigma segment, two waves otherwise.  At G = 4
    the switch lies between w = 496 and w = 497; both sides against the oracle on sampled rows
    (first, last, tile boundaries, random), bf16 bar."""
    B, n, Hq, Hkv, d = 1, 2048, 8, 2, 128
    host, dev = _data(41, B, n, Hq, Hkv, d, "bf16")
    sig_dev, sig = _sigma(42, n)
    q, k, v, _ = dev
    out = ssw.sa_forward(q, k, v, sig_dev, w, causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(43)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 33, n - 2, n - 1],
                                     rng.choice(n, size=40, replace=False)]))
    qh, kh, vh, _ = host
    ref = oracle.sa_rows(qh, kh, vh, sig, w, causal, rows)
    err = _maxerr(out[:, rows], ref, "bf16")
    _say(f"SA alone w={w} causal={causal}: max err {err:.3e}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("vscale", [1e-3, 1e3])
def test_gated_intermediate_across_magnitudes(vscale, causal):
    """The bf16 gated layer keeps g_sa Y_sa between its passes as fp16 of the value times 2^-4:
    normal fp16 for 2^-10 <= |g_sa Y_sa| < 1.05e6, a fixed 2^-20 step below.  V scaled by 1e-3
    puts the outputs around 1e-4, partly below that normal range; V scaled by 1e3 puts them
    around 1e2.  bf16 rounding is relative, so the unit-scale bar is carried to the output's
    scale: max |err| <= 1.5e-2 * max |oracle| (about 1e-5 at the small scale, where a 2^-16 step
    would already use most of it).  Every row."""
    B, n, Hq, Hkv, d, w = 1, 1024, 8, 2, 128, 64
    q, k, v = synth.qkv(71, B, n, Hq, Hkv, d, "bf16")
    g = synth.gates(71, B, n, Hq)
    v = (v.float() * vscale).to(torch.bfloat16)
    sig_dev, sig = _sigma(72, n)
    out = ssw.gated_sa_swa_forward(q.to(DEV), k.to(DEV), v.to(DEV), sig_dev, w, causal, g.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.gated_forward(q, k, v, sig, w, causal, g)
    got = out.float().cpu().numpy().astype(np.float64)
    scale = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    _say(f"gated, V x {vscale:g}, causal={causal}: max |oracle| {scale:.3e}, max err {err:.3e} "
         f"({err / scale:.2e} of it)")
    assert np.isfinite(got).all()
    assert err <= 1.5e-2 * scale, (err, scale)


@pytest.mark.parametrize("w", [448, 449])
def test_gated_d64_build_switch(w):
    """The gated layer's SA pass at d = 64 also has the build with more waves per SIMD (four at
    d = 64), used when a workgroup's band fits its 1024-entry sigma segment; with one query head
    per KV head (G = 1) the switch lies between w = 448 and w = 449.  Both sides of the gated
    layer against the oracle on sampled rows, bf16 bar."""
    B, n, Hq, Hkv, d = 2, 1536, 2, 2, 64
    host, dev = _data(51, B, n, Hq, Hkv, d, "bf16")
    sig_dev, sig = _sigma(52, n)
    q, k, v, g = dev
    out = ssw.gated_sa_swa_forward(q, k, v, sig_dev, w, True, g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(53)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 129, n - 2, n - 1],
                                     rng.choice(n, size=40, replace=False)]))
    qh, kh, vh, gh = host
    ref = oracle.gated_forward(qh, kh, vh, sig, w, True, gh, rows)
    err = _maxerr(out[:, rows], ref, "bf16")
    _say(f"gated d64 w={w}: max err {err:.3e}")
