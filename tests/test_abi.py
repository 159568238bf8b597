"""CPU checks of libssw.so: it loads, exports every symbol include/ssw.h declares, its host-side
permutation generator matches the oracle's bit for bit, and malformed calls are rejected with the
documented status codes before anything reaches the GPU (no compute call is made here)."""

import ctypes
import os
import re

import numpy as np
import pytest

import stochastic_sliding_window_amd as ssw
import synth
from oracle import make_permutation as oracle_perm, inverse_permutation as oracle_inv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssw.h")


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssw_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_symbols()
    assert {"ssw_sa_forward", "ssw_swa_forward", "ssw_gated_sa_swa_forward"} <= set(names)
    lib = ctypes.CDLL(ssw.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("wl", synth.WORKLOADS, ids=lambda w: w.name)
def test_permutation_bit_exact_with_oracle_at_workload_sizes(wl):
    for layer in range(wl.layers):
        seed = synth.sigma_seed(wl.index, layer)
        sigma, inv = ssw.make_permutation(seed, wl.n, with_inverse=True)
        ref = oracle_perm(seed, wl.n)
        assert sigma.dtype == np.int32
        np.testing.assert_array_equal(sigma, ref)
        np.testing.assert_array_equal(inv, oracle_inv(ref))


@pytest.mark.parametrize("n", [0, 1, 2, 3, 17, 1000])
def test_permutation_small_and_extreme_seeds(n):
    for seed in (0, 1, 1234567, 2**64 - 1, 2**63):
        np.testing.assert_array_equal(ssw.make_permutation(seed, n), oracle_perm(seed, n))


def test_inverse_and_check():
    s = ssw.make_permutation(42, 513)
    inv = ssw.inverse_permutation(s)
    np.testing.assert_array_equal(inv[s], np.arange(513))
    assert ssw.check_permutation(s)
    bad = s.copy()
    bad[3] = bad[4]
    assert not ssw.check_permutation(bad)
    assert not ssw.check_permutation(np.array([0, 1, 5], dtype=np.int32))
    assert not ssw.check_permutation(np.array([0, -1, 2], dtype=np.int32))
    with pytest.raises(ssw.SSWError) as e:
        ssw.inverse_permutation(bad)
    assert e.value.status == -5
    assert "permutation" in ssw.last_error()


# ---- argument checking: every case below fails before any HIP call is made --------------------

_lib = ctypes.CDLL(ssw.LIB_PATH)
_FWD_ARGS = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 2 + [ctypes.c_void_p] * 2 + \
    [ctypes.c_int] * 6 + [ctypes.c_void_p]
for _n in ("ssw_sa_forward", "ssw_swa_forward", "ssw_gated_sa_swa_forward"):
    getattr(_lib, _n).argtypes = _FWD_ARGS
    getattr(_lib, _n).restype = ctypes.c_int
_lib.ssw_gated_sa_swa_forward_timed.argtypes = _FWD_ARGS + [ctypes.c_void_p] * 4
_lib.ssw_gated_sa_swa_forward_timed.restype = ctypes.c_int
_lib.ssw_last_error.restype = ctypes.c_char_p

P = 4096  # a fake, 16-byte aligned "device address": never dereferenced in these cases
GOOD = dict(q=P, k=P, v=P, sigma=P, window=8, causal=1, gate=None, out=P,
            B=1, n=64, Hq=4, Hkv=2, d=64, dtype=1)


def _call(fn, **kw):
    a = dict(GOOD)
    a.update(kw)
    extra = (None, None, None, None) if fn.endswith("_timed") else ()
    return getattr(_lib, fn)(a["q"], a["k"], a["v"], a["sigma"], a["window"], a["causal"],
                             a["gate"], a["out"], a["B"], a["n"], a["Hq"], a["Hkv"], a["d"],
                             a["dtype"], None, *extra)


ALL_FWD = ["ssw_sa_forward", "ssw_swa_forward", "ssw_gated_sa_swa_forward",
           "ssw_gated_sa_swa_forward_timed"]


@pytest.mark.parametrize("fn", ALL_FWD)
@pytest.mark.parametrize("kw,status", [
    (dict(window=0), -1),
    (dict(window=-3), -1),
    (dict(causal=2), -1),
    (dict(n=-1), -1),
    (dict(Hkv=0), -1),
    (dict(q=None), -1),
    (dict(out=None), -1),
    (dict(Hq=6, Hkv=4), -2),
    (dict(n=2**30, Hq=8, Hkv=2), -2),
    (dict(n=2**21, Hq=8, Hkv=8, d=128, dtype=0), -2),    # K/V rows past 2^31 bytes
    (dict(d=96), -3),
    (dict(d=256), -3),
    (dict(dtype=7), -3),
    (dict(q=P + 8), -4),
    (dict(out=P + 4), -4),
])
def test_bad_arguments_rejected(fn, kw, status):
    if fn == "ssw_swa_forward":
        kw = dict(kw)
        kw.setdefault("sigma", None)
    assert _call(fn, **kw) == status
    assert _lib.ssw_last_error().decode().startswith(fn)


def test_entry_point_specific_checks():
    assert _call("ssw_sa_forward", sigma=None) == -1
    assert _call("ssw_sa_forward", sigma=P + 2) == -4
    assert _call("ssw_swa_forward", sigma=P) == -1          # SWA takes no permutation
    assert _call("ssw_gated_sa_swa_forward", gate=None) == -1
    assert _call("ssw_gated_sa_swa_forward", gate=P + 1) == -4
    assert _call("ssw_gated_sa_swa_forward_timed", sigma=None) == -1


@pytest.mark.parametrize("fn", ALL_FWD)
def test_empty_calls_are_noops(fn):
    sig = None if fn == "ssw_swa_forward" else P
    for kw in (dict(B=0), dict(n=0)):
        assert _call(fn, q=None, k=None, v=None, out=None, sigma=sig, **kw) == 0


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 8, 2, 64)
    with pytest.raises(TypeError):
        ssw.sa_forward(x, x[:, :, :1], x[:, :, :1], torch.arange(8, dtype=torch.int32), 4, True)


def test_one_hip_runtime_in_process():
    """Importing the binding must leave exactly one HIP runtime mapped (torch's).  A second copy,
    pulled in when libssw.so is loaded before torch, makes every launch fail with "no ROCm-capable
    device" on a GPU host."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import stochastic_sliding_window_amd, torch\n"
        "maps = open('/proc/self/maps').read().splitlines()\n"
        "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n" % ROOT)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip().splitlines()[-1] == "1"


# ---- training entry points: argument checks (no HIP call is reached) ---------------------------

_VP, _I = ctypes.c_void_p, ctypes.c_int
for _n in ("ssw_sa_forward_lse", "ssw_swa_forward_lse"):
    getattr(_lib, _n).argtypes = [_VP] * 4 + [_I] * 2 + [_VP] * 2 + [_I] * 6 + [_VP]
    getattr(_lib, _n).restype = _I
for _n in ("ssw_sa_backward", "ssw_swa_backward"):
    getattr(_lib, _n).argtypes = [_VP] * 4 + [_I] * 2 + [_VP] * 9 + [_I] * 7 + [_VP]
    getattr(_lib, _n).restype = _I
_lib.ssw_gated_sa_swa_forward_train.argtypes = [_VP] * 4 + [_I] * 2 + [_VP] * 6 + [_I] * 6 + [_VP]
_lib.ssw_gated_sa_swa_forward_train.restype = _I
_lib.ssw_gated_sa_swa_backward.argtypes = [_VP] * 4 + [_I] * 2 + [_VP] * 11 + [_I] * 6 + [_VP]
_lib.ssw_gated_sa_swa_backward.restype = _I

BWD_GOOD = dict(GOOD, out=P, lse=P, dout=P, dq=P, dk=P, dv=P, dgate=None, delta=P, accumulate=0)


def _call_bwd(fn, **kw):
    a = dict(BWD_GOOD)
    if fn == "ssw_swa_backward":
        a["sigma"] = None
    a.update(kw)
    return getattr(_lib, fn)(a["q"], a["k"], a["v"], a["sigma"], a["window"], a["causal"],
                             a["gate"], a["out"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                             a["dgate"], a["delta"], a["accumulate"], a["B"], a["n"], a["Hq"],
                             a["Hkv"], a["d"], a["dtype"], None)


@pytest.mark.parametrize("fn", ["ssw_sa_backward", "ssw_swa_backward"])
@pytest.mark.parametrize("kw,status", [
    (dict(window=0), -1),
    (dict(causal=3), -1),
    (dict(accumulate=2), -1),
    (dict(dout=None), -1),
    (dict(lse=None), -1),
    (dict(delta=None), -1),
    (dict(dk=None), -1),
    (dict(Hq=6, Hkv=4), -2),
    (dict(dtype=0), -3),           # the backward takes bf16 only
    (dict(d=80), -3),
    (dict(dq=P + 8), -4),
    (dict(lse=P + 2), -4),
    (dict(gate=P + 1), -4),
])
def test_backward_bad_arguments_rejected(fn, kw, status):
    assert _call_bwd(fn, **kw) == status
    assert _lib.ssw_last_error().decode().startswith(fn)


def test_backward_entry_point_specific_checks():
    assert _call_bwd("ssw_sa_backward", sigma=None) == -1
    assert _call_bwd("ssw_swa_backward", sigma=P) == -1
    assert _call_bwd("ssw_sa_backward", B=0, q=None, k=None, v=None, out=None) == 0


def test_forward_lse_checks():
    args = lambda sig, lse, dtype=1: (P, P, P, sig, 8, 1, P, lse, 1, 64, 4, 2, 64, dtype, None)
    assert _lib.ssw_sa_forward_lse(*args(None, P)) == -1
    assert _lib.ssw_sa_forward_lse(*args(P, None)) == -1
    assert _lib.ssw_sa_forward_lse(*args(P, P + 2)) == -4
    assert _lib.ssw_swa_forward_lse(*args(P, P)) == -1


def test_gated_training_checks():
    fwd = lambda **kw: _lib.ssw_gated_sa_swa_forward_train(
        P, P, P, kw.get("sigma", P), 8, 1, kw.get("gates", P), P, kw.get("y_sa", P), P, P, P,
        1, 64, 4, 2, 64, kw.get("dtype", 1), None)
    assert fwd(gates=None) == -1
    assert fwd(y_sa=None) == -1
    assert fwd(y_sa=P + 8) == -4
    assert fwd(dtype=0) == -3
    bwd = lambda **kw: _lib.ssw_gated_sa_swa_backward(
        P, P, P, kw.get("sigma", P), 8, 1, P, P, P, kw.get("y_swa", P), P, P, P, P, P,
        kw.get("dgates", None), P, 1, 64, 4, 2, 64, kw.get("dtype", 1), None)
    assert bwd(sigma=None) == -1
    assert bwd(y_swa=None) == -1
    assert bwd(dgates=P + 1) == -4
    assert bwd(dtype=0) == -3


def test_gated_backward_noalloc_checks():
    """The backward that allocates nothing: the same argument checks (made before any HIP call),
    and its size limit, B * n * Hq <= 2^22 (the library's own Delta array)."""
    fn = _lib.ssw_gated_sa_swa_backward_noalloc
    fn.argtypes = [_VP] * 4 + [_I] * 2 + [_VP] * 10 + [_I] * 6 + [_VP]
    fn.restype = _I
    bwd = lambda **kw: fn(
        P, P, P, kw.get("sigma", P), 8, 1, P, P, P, kw.get("y_swa", P), P, P, P, P, P,
        kw.get("dgates", None), kw.get("B", 1), kw.get("n", 64), kw.get("Hq", 4), 2, 64,
        kw.get("dtype", 1), None)
    assert bwd(sigma=None) == -1
    assert bwd(y_swa=None) == -1
    assert bwd(dgates=P + 1) == -4
    assert bwd(dtype=0) == -3
    assert bwd(B=0) == 0 and bwd(n=0) == 0
    assert bwd(B=2, n=65536, Hq=34) == -2
    assert "Delta array" in ssw.last_error()


# ---- decode entry points -----------------------------------------------------------------------

for _n in ("ssw_sa_decode", "ssw_swa_decode", "ssw_gated_sa_swa_decode"):
    getattr(_lib, _n).argtypes = [_VP] * 6 + [_I] + [_VP] * 2 + [_I] * 6 + [_VP]
    getattr(_lib, _n).restype = _I

DEC_GOOD = dict(q=P, k=P, v=P, sigma=P, inv=P, pos=P, window=8, gate=P, out=P, B=2, n=64, Hq=8,
                Hkv=2, d=128, dtype=1)


def _call_dec(fn, **kw):
    a = dict(DEC_GOOD)
    if fn == "ssw_swa_decode":
        a.update(sigma=None, inv=None)
    a.update(kw)
    return getattr(_lib, fn)(a["q"], a["k"], a["v"], a["sigma"], a["inv"], a["pos"], a["window"],
                             a["gate"], a["out"], a["B"], a["n"], a["Hq"], a["Hkv"], a["d"],
                             a["dtype"], None)


@pytest.mark.parametrize("fn", ["ssw_sa_decode", "ssw_swa_decode", "ssw_gated_sa_swa_decode"])
@pytest.mark.parametrize("kw,status", [
    (dict(window=0), -1),
    (dict(n=0), -1),
    (dict(pos=None), -1),
    (dict(out=None), -1),
    (dict(Hq=6, Hkv=4), -2),
    (dict(Hq=32, Hkv=2), -2),      # more than 8 query heads per KV head
    (dict(d=32), -3),
    (dict(dtype=5), -3),
    (dict(q=P + 8), -4),
    (dict(pos=P + 2), -4),
])
def test_decode_bad_arguments_rejected(fn, kw, status):
    assert _call_dec(fn, **kw) == status
    assert _lib.ssw_last_error().decode().startswith(fn)


def test_decode_specific_checks():
    assert _call_dec("ssw_sa_decode", sigma=None) == -1
    assert _call_dec("ssw_sa_decode", inv=None) == -1
    assert _call_dec("ssw_swa_decode", sigma=P) == -1
    assert _call_dec("ssw_gated_sa_swa_decode", gate=None) == -1
    assert _call_dec("ssw_sa_decode", B=0, q=None) == 0


def test_strided_sigma_checks():
    for fn in ("ssw_sa_forward_ex", "ssw_gated_sa_swa_forward_ex"):
        f = getattr(_lib, fn)
        f.argtypes = [_VP] * 4 + [ctypes.c_int64] * 2 + [_I] * 2 + [_VP] * 2 + [_I] * 6 + [_VP]
        f.restype = _I
        args = lambda sig=P, sb=0, sh=0, gate=P: (P, P, P, sig, sb, sh, 8, 1, gate, P, 1, 64, 4, 2,
                                                  64, 1, None)
        assert f(*args(sig=None)) == -1
        assert f(*args(sb=-1)) == -1
        assert f(*args(sh=-64)) == -1
        assert f(*args(sig=P + 2)) == -4
    assert _lib.ssw_gated_sa_swa_forward_ex(P, P, P, P, 0, 0, 8, 1, None, P, 1, 64, 4, 2, 64, 1,
                                            None) == -1


def test_gate_projection_checks():
    f = _lib.ssw_gate_projection
    f.argtypes = [_VP] * 4 + [_I] * 4 + [_VP]
    f.restype = _I
    assert f(P, P, None, P, -1, 64, 4, 1, None) == -1
    assert f(P, P, None, P, 10, 64, 4, 0, None) == -3
    assert f(P, P, None, P, 10, 40, 4, 1, None) == -2       # Hm not a multiple of 16
    assert f(P, P, None, P, 10, 64, 65, 1, None) == -2      # Hq > 64
    assert f(None, P, None, P, 10, 64, 4, 1, None) == -1
    assert f(P + 8, P, None, P, 10, 64, 4, 1, None) == -4
    assert f(P, P, None, P, 0, 64, 4, 1, None) == 0
