"""Stochastic Attention (SA), SWA and gated SA+SWA for AMD MI355X (gfx950): forward and backward.

Thin ctypes binding over the C ABI of ``libssw.so`` (declared in ``include/ssw.h``).  Every
function here only marshals arguments -- tensor checks, device pointers, the current HIP stream
-- and calls the library; all arithmetic runs in the library's HIP kernels (or, for the
permutation helpers, its host C++ code).  PyTorch supplies device memory and streams.

The functions keep the C names without the ``ssw_`` prefix:

    sa_forward(q, k, v, sigma, window, causal, gate=None, out=None)
    swa_forward(q, k, v, window, causal, gate=None, out=None)
    gated_sa_swa_forward(q, k, v, sigma, window, causal, gates, out=None, events=None)
    make_permutation(seed, n) / inverse_permutation(sigma) / check_permutation(sigma)
    neighbor_mask(sigma, n, window, causal)

Training (bf16):

    sa_forward_lse(q, k, v, sigma, window, causal, out=None, lse=None) -> (out, lse)
    swa_forward_lse(q, k, v, window, causal, out=None, lse=None) -> (out, lse)
    sa_backward(q, k, v, sigma, window, causal, out, lse, dout, gate=None, ...) -> (dq, dk, dv, dgate)
    swa_backward(q, k, v, window, causal, out, lse, dout, gate=None, ...) -> (dq, dk, dv, dgate)
    gated_sa_swa_forward_train(q, k, v, sigma, window, causal, gates) -> (out, saved)
    gated_sa_swa_backward(q, k, v, sigma, window, causal, gates, saved, dout) -> (dq, dk, dv, dgates)
    gated_sa_swa_backward_noalloc(q, k, v, sigma, window, causal, gates, saved, dout, dq, dk, dv,
                                  dgates=None)   (allocates nothing: Delta in the library's array)

Variant: one sigma per batch row and/or KV head (sigma [B, n], [Hkv, n] or [B, Hkv, n]):

    sa_forward_ex(q, k, v, sigmas, window, causal, gate=None, out=None)
    gated_sa_swa_forward_ex(q, k, v, sigmas, window, causal, gates, out=None)

Gate projections (g = sigmoid(x w_t^T + b) into the [2, B, n, Hq] gates layout):

    gate_projection(x, w_t, bias=None, Hq=None, out=None)

Decode (one new token per batch row over a KV cache):

    sa_decode(q, k_cache, v_cache, sigma, inv_sigma, pos, window, gate=None, out=None)
    swa_decode(q, k_cache, v_cache, pos, window, gate=None, out=None)
    gated_sa_swa_decode(q, k_cache, v_cache, sigma, inv_sigma, pos, window, gates, out=None)

There is no fallback: if ``libssw.so`` has not been built, importing this package raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
# torch first: it loads its bundled HIP runtime under the unversioned name libamdhip64.so.  If
# libssw.so were loaded first, its libamdhip64.so.7 would come from /opt/rocm and torch would then
# load a second HIP runtime into the process, whose device list the library's launches do not
# share ("no ROCm-capable device").  Loaded after torch, libssw.so binds to torch's runtime (same
# soname), so tensors, streams and events are all one runtime's objects.
import torch  # noqa: F401  (import order matters, see above)

__all__ = [
    "SSWError", "LIB_PATH", "sa_forward", "swa_forward", "gated_sa_swa_forward",
    "make_permutation", "inverse_permutation", "check_permutation", "neighbor_mask",
    "last_error", "F32", "BF16", "sa_forward_lse", "swa_forward_lse", "sa_backward",
    "swa_backward", "gated_sa_swa_forward_train", "gated_sa_swa_backward",
    "gated_sa_swa_backward_noalloc", "sa_decode",
    "swa_decode", "gated_sa_swa_decode", "sa_forward_ex", "gated_sa_swa_forward_ex",
    "receptive_field_coverage", "gate_projection",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# SSW_LIBRARY may name another build of the same library (e.g. one compiled with different tile
# constants); by default the in-tree build is used.
LIB_PATH = os.environ.get("SSW_LIBRARY") or os.path.join(_PKG_DIR, "libssw.so")

F32 = 0
BF16 = 1

_STATUS = {
    0: "SSW_OK", -1: "SSW_EINVAL", -2: "SSW_ESHAPE", -3: "SSW_EDTYPE", -4: "SSW_EALIGN",
    -5: "SSW_ENOTPERM", -6: "SSW_EHIP",
}


class SSWError(RuntimeError):
    """A libssw call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {message}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first with "
            "`python stochastic_sliding_window_amd/build.py` (needs ROCm hipcc)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32p, i32p = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    fwd = [vp, vp, vp, i32p, i32, i32, f32p, vp, i32, i32, i32, i32, i32, i32, vp]
    for name in ("ssw_sa_forward", "ssw_swa_forward", "ssw_gated_sa_swa_forward"):
        fn = getattr(lib, name)
        fn.argtypes = fwd
        fn.restype = ctypes.c_int
    lib.ssw_gated_sa_swa_forward_timed.argtypes = fwd + [vp, vp, vp, vp]
    lib.ssw_gated_sa_swa_forward_timed.restype = ctypes.c_int
    fwd_lse = [vp, vp, vp, i32p, i32, i32, vp, f32p, i32, i32, i32, i32, i32, i32, vp]
    for name in ("ssw_sa_forward_lse", "ssw_swa_forward_lse"):
        fn = getattr(lib, name)
        fn.argtypes = fwd_lse
        fn.restype = ctypes.c_int
    bwd = [vp, vp, vp, i32p, i32, i32, f32p, vp, f32p, vp, vp, vp, vp, f32p, f32p, i32,
           i32, i32, i32, i32, i32, i32, vp]
    for name in ("ssw_sa_backward", "ssw_swa_backward"):
        fn = getattr(lib, name)
        fn.argtypes = bwd
        fn.restype = ctypes.c_int
    lib.ssw_gated_sa_swa_forward_train.argtypes = [vp, vp, vp, i32p, i32, i32, f32p, vp, vp, f32p,
                                                   vp, f32p, i32, i32, i32, i32, i32, i32, vp]
    lib.ssw_gated_sa_swa_forward_train.restype = ctypes.c_int
    lib.ssw_gated_sa_swa_backward.argtypes = [vp, vp, vp, i32p, i32, i32, f32p, vp, f32p, vp, f32p,
                                              vp, vp, vp, vp, f32p, f32p, i32, i32, i32, i32, i32,
                                              i32, vp]
    lib.ssw_gated_sa_swa_backward.restype = ctypes.c_int
    lib.ssw_gated_sa_swa_backward_noalloc.argtypes = [vp, vp, vp, i32p, i32, i32, f32p, vp, f32p,
                                                      vp, f32p, vp, vp, vp, vp, f32p, i32, i32,
                                                      i32, i32, i32, i32, vp]
    lib.ssw_gated_sa_swa_backward_noalloc.restype = ctypes.c_int
    dec = [vp, vp, vp, i32p, i32p, i32p, i32, f32p, vp, i32, i32, i32, i32, i32, i32, vp]
    for name in ("ssw_sa_decode", "ssw_swa_decode", "ssw_gated_sa_swa_decode"):
        fn = getattr(lib, name)
        fn.argtypes = dec
        fn.restype = ctypes.c_int
    i64 = ctypes.c_int64
    for name in ("ssw_sa_forward_ex", "ssw_gated_sa_swa_forward_ex"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, i32p, i64, i64, i32, i32, f32p, vp, i32, i32, i32, i32, i32,
                       i32, vp]
        fn.restype = ctypes.c_int
    lib.ssw_gate_projection.argtypes = [vp, vp, f32p, f32p, i32, i32, i32, i32, vp]
    lib.ssw_gate_projection.restype = ctypes.c_int
    lib.ssw_receptive_field_coverage.argtypes = [i32, i32, i32, vp, i32, i32, vp]
    lib.ssw_receptive_field_coverage.restype = ctypes.c_int
    lib.ssw_make_permutation.argtypes = [ctypes.c_uint64, i32, i32p, i32p]
    lib.ssw_make_permutation.restype = ctypes.c_int
    lib.ssw_inverse_permutation.argtypes = [i32p, i32, i32p]
    lib.ssw_inverse_permutation.restype = ctypes.c_int
    lib.ssw_check_permutation.argtypes = [i32p, i32]
    lib.ssw_check_permutation.restype = ctypes.c_int
    lib.ssw_neighbor_mask.argtypes = [i32p, i32, i32, i32, vp, vp]
    lib.ssw_neighbor_mask.restype = ctypes.c_int
    lib.ssw_last_error.argtypes = []
    lib.ssw_last_error.restype = ctypes.c_char_p
    return lib


_lib = _load()


def last_error() -> str:
    return _lib.ssw_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise SSWError(status, last_error())


# ------------------------------------------------------------------------------------------
# host helpers
# ------------------------------------------------------------------------------------------

def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def make_permutation(seed: int, n: int, with_inverse: bool = False):
    """sigma (int32[n]) for one layer from the seeded generator; optionally also sigma^-1."""
    sigma = np.empty(n, dtype=np.int32)
    inv = np.empty(n, dtype=np.int32) if with_inverse else None
    _check(_lib.ssw_make_permutation(ctypes.c_uint64(seed & (2**64 - 1)), n, _np_ptr(sigma),
                                     _np_ptr(inv) if inv is not None else None))
    return (sigma, inv) if with_inverse else sigma


def inverse_permutation(sigma) -> np.ndarray:
    s = np.ascontiguousarray(np.asarray(sigma, dtype=np.int32))
    inv = np.empty_like(s)
    _check(_lib.ssw_inverse_permutation(_np_ptr(s), s.shape[0], _np_ptr(inv)))
    return inv


def receptive_field_coverage(n: int, window: int, seeds, mode: str = "sa",
                             causal: bool = True) -> np.ndarray:
    """Coverage after each layer (ssw_receptive_field_coverage); one seed per layer, mode 'sa',
    'swa' or 'gated'."""
    modes = {"sa": 0, "swa": 1, "gated": 2}
    sd = np.ascontiguousarray(np.asarray([int(x) & (2**64 - 1) for x in seeds], dtype=np.uint64))
    out = np.empty(sd.shape[0], dtype=np.float64)
    _check(_lib.ssw_receptive_field_coverage(int(n), int(window), sd.shape[0], _np_ptr(sd),
                                             modes[mode], int(bool(causal)), _np_ptr(out)))
    return out


def check_permutation(sigma) -> bool:
    s = np.ascontiguousarray(np.asarray(sigma, dtype=np.int32))
    st = _lib.ssw_check_permutation(_np_ptr(s), s.shape[0])
    if st == -5:
        return False
    _check(st)
    return True


# ------------------------------------------------------------------------------------------
# device entry points
# ------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _stream_handle(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev_ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _prep(q, k, v, out):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a device tensor")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, n, H, d] tensor")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if k.shape != v.shape or k.shape[:2] != q.shape[:2] or k.shape[3] != q.shape[3]:
        raise ValueError("k and v must be [B, n, Hkv, d] matching q [B, n, Hq, d]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous device tensor shaped and typed like q")
    return out


def _prep_sigma(sigma, n, device):
    torch = _torch()
    if not isinstance(sigma, torch.Tensor) or sigma.dtype != torch.int32 or \
            sigma.shape != (n,) or not sigma.is_contiguous() or sigma.device != device:
        raise ValueError("sigma must be a contiguous int32 [n] tensor on the same device as q")
    return sigma


def _prep_gate(gate, shape, device):
    torch = _torch()
    if gate is None:
        return None
    if gate.dtype != torch.float32 or tuple(gate.shape) != tuple(shape) or \
            not gate.is_contiguous() or gate.device != device:
        raise ValueError(f"gate must be a contiguous float32 {tuple(shape)} tensor on q's device")
    return gate


def sa_forward(q, k, v, sigma, window: int, causal: bool, gate=None, out=None):
    """Stochastic Attention forward (ssw_sa_forward): out[b, sigma[p], h] = window attention of
    slot p in the permuted space, times ``gate`` [B, n, Hq] if given."""
    out = _prep(q, k, v, out)
    B, n, Hq, d = q.shape
    sigma = _prep_sigma(sigma, n, q.device)
    gate = _prep_gate(gate, (B, n, Hq), q.device)
    _check(_lib.ssw_sa_forward(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sigma), int(window),
                               int(bool(causal)), _dev_ptr(gate), _dev_ptr(out), B, n, Hq,
                               k.shape[2], d, _dtype_code(q), _stream_handle(q)))
    return out


def swa_forward(q, k, v, window: int, causal: bool, gate=None, out=None):
    """Plain sliding-window attention forward (ssw_swa_forward)."""
    out = _prep(q, k, v, out)
    B, n, Hq, d = q.shape
    gate = _prep_gate(gate, (B, n, Hq), q.device)
    _check(_lib.ssw_swa_forward(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), None, int(window),
                                int(bool(causal)), _dev_ptr(gate), _dev_ptr(out), B, n, Hq,
                                k.shape[2], d, _dtype_code(q), _stream_handle(q)))
    return out


def gated_sa_swa_forward(q, k, v, sigma, window: int, causal: bool, gates, out=None, events=None):
    """Y = g_sa * SA + g_swa * SWA with gates [2, B, n, Hq] (ssw_gated_sa_swa_forward).

    ``events``: optional (swa_start, swa_end, sa_start, sa_end) torch.cuda.Event 4-tuple attached
    to the two kernels' dispatches (ssw_gated_sa_swa_forward_timed); each must have been recorded
    once already so that its HIP event exists.
    """
    out = _prep(q, k, v, out)
    B, n, Hq, d = q.shape
    sigma = _prep_sigma(sigma, n, q.device)
    if gates is None:
        raise ValueError("gates are required")
    gates = _prep_gate(gates, (2, B, n, Hq), q.device)
    args = (_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sigma), int(window), int(bool(causal)),
            _dev_ptr(gates), _dev_ptr(out), B, n, Hq, k.shape[2], d, _dtype_code(q),
            _stream_handle(q))
    if events is None:
        _check(_lib.ssw_gated_sa_swa_forward(*args))
    else:
        if len(events) != 4:
            raise ValueError("events: (swa_start, swa_end, sa_start, sa_end)")
        handles = []
        for e in events:
            if e is None:
                handles.append(None)
                continue
            h = e.cuda_event
            if not h:
                raise ValueError("record each event once before passing it (its HIP event is lazy)")
            handles.append(ctypes.c_void_p(h))
        _check(_lib.ssw_gated_sa_swa_forward_timed(*args, *handles))
    return out


def neighbor_mask(sigma, n: int, window: int, causal: bool, device=None):
    """uint32 [n, ceil(n/32)] device bitmask of the neighbour sets (ssw_neighbor_mask).

    sigma: int32 [n] device tensor, or None for SWA.
    """
    torch = _torch()
    if sigma is not None:
        device = sigma.device
        sigma = _prep_sigma(sigma, n, device)
    words = (n + 31) // 32
    bits = torch.empty((n, words), dtype=torch.int32, device=device)
    _check(_lib.ssw_neighbor_mask(_dev_ptr(sigma), n, int(window), int(bool(causal)),
                                  _dev_ptr(bits), ctypes.c_void_p(
                                      torch.cuda.current_stream(bits.device).cuda_stream)))
    return bits


# ------------------------------------------------------------------------------------------
# training: forward with log-sum-exp, backward
# ------------------------------------------------------------------------------------------

def _prep_rows(t, shape, dtype, device, name):
    """A given output/scratch tensor must be contiguous, on q's device, of the given shape/dtype."""
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype != dtype or \
            not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous {dtype} {tuple(shape)} tensor on q's device")
    return t


def _prep_like(t, ref, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.shape != ref.shape or t.dtype != ref.dtype or \
            not t.is_contiguous() or t.device != ref.device:
        raise ValueError(f"{name} must be a contiguous tensor shaped and typed like {tuple(ref.shape)}")
    return t


def _forward_lse(fn, q, k, v, sigma, window, causal, out, lse):
    torch = _torch()
    out = _prep(q, k, v, out)
    B, n, Hq, d = q.shape
    lse = _prep_rows(lse, (B, n, Hq), torch.float32, q.device, "lse")
    _check(fn(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sigma), int(window),
              int(bool(causal)), _dev_ptr(out), _dev_ptr(lse), B, n, Hq, k.shape[2], d,
              _dtype_code(q), _stream_handle(q)))
    return out, lse


def sa_forward_lse(q, k, v, sigma, window: int, causal: bool, out=None, lse=None):
    """SA forward without gate that also returns each row's log-sum-exp (ssw_sa_forward_lse)."""
    sigma = _prep_sigma(sigma, q.shape[1], q.device)
    return _forward_lse(_lib.ssw_sa_forward_lse, q, k, v, sigma, window, causal, out, lse)


def swa_forward_lse(q, k, v, window: int, causal: bool, out=None, lse=None):
    """SWA forward that also returns each row's log-sum-exp (ssw_swa_forward_lse)."""
    return _forward_lse(_lib.ssw_swa_forward_lse, q, k, v, None, window, causal, out, lse)


def _backward(fn, q, k, v, sigma, window, causal, out, lse, dout, gate, dq, dk, dv, dgate,
              delta, accumulate, want_dgate):
    torch = _torch()
    _prep(q, k, v, None if out is None else out)
    B, n, Hq, d = q.shape
    out = _prep_like(out, q, "out")
    dout = _prep_like(dout, q, "dout")
    lse = _prep_rows(lse, (B, n, Hq), torch.float32, q.device, "lse") if lse is not None else None
    if lse is None:
        raise ValueError("lse is required")
    gate = _prep_gate(gate, (B, n, Hq), q.device)
    if accumulate and (dq is None or dk is None or dv is None):
        raise ValueError("accumulate needs dq, dk and dv to add to")
    dq = _prep_like(dq, q, "dq") if dq is not None else torch.empty_like(q)
    dk = _prep_like(dk, k, "dk") if dk is not None else torch.empty_like(k)
    dv = _prep_like(dv, v, "dv") if dv is not None else torch.empty_like(v)
    if dgate is None and want_dgate:
        dgate = torch.empty((B, n, Hq), dtype=torch.float32, device=q.device)
    elif dgate is not None:
        dgate = _prep_rows(dgate, (B, n, Hq), torch.float32, q.device, "dgate")
    delta = _prep_rows(delta, (B, n, Hq), torch.float32, q.device, "delta")
    _check(fn(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sigma), int(window),
              int(bool(causal)), _dev_ptr(gate), _dev_ptr(out), _dev_ptr(lse), _dev_ptr(dout),
              _dev_ptr(dq), _dev_ptr(dk), _dev_ptr(dv), _dev_ptr(dgate), _dev_ptr(delta),
              int(bool(accumulate)), B, n, Hq, k.shape[2], d, _dtype_code(q), _stream_handle(q)))
    return dq, dk, dv, dgate


def sa_backward(q, k, v, sigma, window: int, causal: bool, out, lse, dout, gate=None, dq=None,
                dk=None, dv=None, dgate=None, delta=None, accumulate=False, want_dgate=True):
    """Gradients of y = gate * SA(q, k, v) given dout = dL/dy (ssw_sa_backward).

    out and lse come from sa_forward_lse.  Returns (dq, dk, dv, dgate); with accumulate=True the
    gradients are added to the given dq, dk, dv.
    """
    sigma = _prep_sigma(sigma, q.shape[1], q.device)
    return _backward(_lib.ssw_sa_backward, q, k, v, sigma, window, causal, out, lse, dout, gate,
                     dq, dk, dv, dgate, delta, accumulate, want_dgate)


def swa_backward(q, k, v, window: int, causal: bool, out, lse, dout, gate=None, dq=None, dk=None,
                 dv=None, dgate=None, delta=None, accumulate=False, want_dgate=True):
    """Gradients of y = gate * SWA(q, k, v) given dout (ssw_swa_backward)."""
    return _backward(_lib.ssw_swa_backward, q, k, v, None, window, causal, out, lse, dout, gate,
                     dq, dk, dv, dgate, delta, accumulate, want_dgate)


def gated_sa_swa_forward_train(q, k, v, sigma, window: int, causal: bool, gates, out=None,
                               saved=None):
    """Training forward of the gated layer (ssw_gated_sa_swa_forward_train).

    Returns (out, saved) with saved = (y_sa, lse_sa, y_swa, lse_swa) for the backward.
    """
    torch = _torch()
    out = _prep(q, k, v, out)
    B, n, Hq, d = q.shape
    sigma = _prep_sigma(sigma, n, q.device)
    if gates is None:
        raise ValueError("gates are required")
    gates = _prep_gate(gates, (2, B, n, Hq), q.device)
    if saved is None:
        saved = (torch.empty_like(q), torch.empty((B, n, Hq), dtype=torch.float32, device=q.device),
                 torch.empty_like(q), torch.empty((B, n, Hq), dtype=torch.float32, device=q.device))
    y_sa, lse_sa, y_swa, lse_swa = saved
    y_sa, y_swa = _prep_like(y_sa, q, "y_sa"), _prep_like(y_swa, q, "y_swa")
    lse_sa = _prep_rows(lse_sa, (B, n, Hq), torch.float32, q.device, "lse_sa")
    lse_swa = _prep_rows(lse_swa, (B, n, Hq), torch.float32, q.device, "lse_swa")
    _check(_lib.ssw_gated_sa_swa_forward_train(
        _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sigma), int(window), int(bool(causal)),
        _dev_ptr(gates), _dev_ptr(out), _dev_ptr(y_sa), _dev_ptr(lse_sa), _dev_ptr(y_swa),
        _dev_ptr(lse_swa), B, n, Hq, k.shape[2], d, _dtype_code(q), _stream_handle(q)))
    return out, (y_sa, lse_sa, y_swa, lse_swa)


def gated_sa_swa_backward(q, k, v, sigma, window: int, causal: bool, gates, saved, dout, dq=None,
                          dk=None, dv=None, dgates=None, delta=None, want_dgates=True):
    """Gradients of the gated layer (ssw_gated_sa_swa_backward); saved from the training forward.

    Returns (dq, dk, dv, dgates) with dgates [2, B, n, Hq] (or None if want_dgates is False).
    """
    torch = _torch()
    _prep(q, k, v, None)
    B, n, Hq, d = q.shape
    sigma = _prep_sigma(sigma, n, q.device)
    gates = _prep_gate(gates, (2, B, n, Hq), q.device)
    if gates is None:
        raise ValueError("gates are required")
    y_sa, lse_sa, y_swa, lse_swa = saved
    y_sa, y_swa = _prep_like(y_sa, q, "y_sa"), _prep_like(y_swa, q, "y_swa")
    lse_sa = _prep_rows(lse_sa, (B, n, Hq), torch.float32, q.device, "lse_sa")
    lse_swa = _prep_rows(lse_swa, (B, n, Hq), torch.float32, q.device, "lse_swa")
    dout = _prep_like(dout, q, "dout")
    dq = _prep_like(dq, q, "dq") if dq is not None else torch.empty_like(q)
    dk = _prep_like(dk, k, "dk") if dk is not None else torch.empty_like(k)
    dv = _prep_like(dv, v, "dv") if dv is not None else torch.empty_like(v)
    if dgates is None and want_dgates:
        dgates = torch.empty((2, B, n, Hq), dtype=torch.float32, device=q.device)
    elif dgates is not None:
        dgates = _prep_rows(dgates, (2, B, n, Hq), torch.float32, q.device, "dgates")
    delta = _prep_rows(delta, (B, n, Hq), torch.float32, q.device, "delta")
    _check(_lib.ssw_gated_sa_swa_backward(
        _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sigma), int(window), int(bool(causal)),
        _dev_ptr(gates), _dev_ptr(y_sa), _dev_ptr(lse_sa), _dev_ptr(y_swa), _dev_ptr(lse_swa),
        _dev_ptr(dout), _dev_ptr(dq), _dev_ptr(dk), _dev_ptr(dv), _dev_ptr(dgates),
        _dev_ptr(delta), B, n, Hq, k.shape[2], d, _dtype_code(q), _stream_handle(q)))
    return dq, dk, dv, dgates


def gated_sa_swa_backward_noalloc(q, k, v, sigma, window: int, causal: bool, gates, saved, dout,
                                  dq, dk, dv, dgates=None):
    """ssw_gated_sa_swa_backward_noalloc: the gated layer's backward with Delta in the library's
    own device array, so the call allocates nothing (dq, dk, dv and, if wanted, dgates are the
    caller's; B * n * Hq <= 2^22).  Returns (dq, dk, dv, dgates)."""
    torch = _torch()
    _prep(q, k, v, None)
    B, n, Hq, d = q.shape
    sigma = _prep_sigma(sigma, n, q.device)
    gates = _prep_gate(gates, (2, B, n, Hq), q.device)
    if gates is None:
        raise ValueError("gates are required")
    y_sa, lse_sa, y_swa, lse_swa = saved
    y_sa, y_swa = _prep_like(y_sa, q, "y_sa"), _prep_like(y_swa, q, "y_swa")
    lse_sa = _prep_rows(lse_sa, (B, n, Hq), torch.float32, q.device, "lse_sa")
    lse_swa = _prep_rows(lse_swa, (B, n, Hq), torch.float32, q.device, "lse_swa")
    dout = _prep_like(dout, q, "dout")
    dq, dk, dv = _prep_like(dq, q, "dq"), _prep_like(dk, k, "dk"), _prep_like(dv, v, "dv")
    if dgates is not None:
        dgates = _prep_rows(dgates, (2, B, n, Hq), torch.float32, q.device, "dgates")
    _check(_lib.ssw_gated_sa_swa_backward_noalloc(
        _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sigma), int(window), int(bool(causal)),
        _dev_ptr(gates), _dev_ptr(y_sa), _dev_ptr(lse_sa), _dev_ptr(y_swa), _dev_ptr(lse_swa),
        _dev_ptr(dout), _dev_ptr(dq), _dev_ptr(dk), _dev_ptr(dv), _dev_ptr(dgates), B, n, Hq,
        k.shape[2], d, _dtype_code(q), _stream_handle(q)))
    return dq, dk, dv, dgates


# ------------------------------------------------------------------------------------------
# decode over a KV cache
# ------------------------------------------------------------------------------------------

def _decode(fn, q, k_cache, v_cache, sigma, inv_sigma, pos, window, gate, gate_shape, out):
    torch = _torch()
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous device tensor")
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, Hq, d] and the caches [B, n_max, Hkv, d]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share a dtype")
    B, Hq, d = q.shape
    n_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[0] != B or k_cache.shape[3] != d:
        raise ValueError("cache shape does not match q")
    if sigma is not None:
        sigma = _prep_sigma(sigma, n_max, q.device)
        inv_sigma = _prep_sigma(inv_sigma, n_max, q.device)
    if not isinstance(pos, torch.Tensor) or pos.dtype != torch.int32 or pos.shape != (B,) or \
            pos.device != q.device or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 [B] tensor on q's device")
    gate = _prep_gate(gate, gate_shape(B, Hq), q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        out = _prep_like(out, q, "out")
    _check(fn(_dev_ptr(q), _dev_ptr(k_cache), _dev_ptr(v_cache), _dev_ptr(sigma),
              _dev_ptr(inv_sigma), _dev_ptr(pos), int(window), _dev_ptr(gate), _dev_ptr(out), B,
              n_max, Hq, Hkv, d, _dtype_code(q), _stream_handle(q)))
    return out


def sa_decode(q, k_cache, v_cache, sigma, inv_sigma, pos, window: int, gate=None, out=None):
    """One SA decode step per batch row (ssw_sa_decode): row pos[b] of causal SA over n_max."""
    return _decode(_lib.ssw_sa_decode, q, k_cache, v_cache, sigma, inv_sigma, pos, window, gate,
                   lambda B, H: (B, H), out)


def swa_decode(q, k_cache, v_cache, pos, window: int, gate=None, out=None):
    """One SWA decode step per batch row (ssw_swa_decode)."""
    return _decode(_lib.ssw_swa_decode, q, k_cache, v_cache, None, None, pos, window, gate,
                   lambda B, H: (B, H), out)


def gated_sa_swa_decode(q, k_cache, v_cache, sigma, inv_sigma, pos, window: int, gates, out=None):
    """g_sa * SA step + g_swa * SWA step, gates [2, B, Hq] (ssw_gated_sa_swa_decode)."""
    if gates is None:
        raise ValueError("gates are required")
    return _decode(_lib.ssw_gated_sa_swa_decode, q, k_cache, v_cache, sigma, inv_sigma, pos,
                   window, gates, lambda B, H: (2, B, H), out)


# ------------------------------------------------------------------------------------------
# variant: one sigma per batch row and/or KV head
# ------------------------------------------------------------------------------------------

def _sigma_strides(sigmas, B, n, Hkv, device):
    """(batch stride, head stride) of a sigma tensor [n], [B, n], [Hkv, n] or [B, Hkv, n]."""
    torch = _torch()
    if not isinstance(sigmas, torch.Tensor) or sigmas.dtype != torch.int32 or \
            not sigmas.is_contiguous() or sigmas.device != device or sigmas.shape[-1] != n:
        raise ValueError("sigmas must be a contiguous int32 tensor [..., n] on q's device")
    shape = tuple(sigmas.shape[:-1])
    if shape == ():
        return 0, 0
    if shape == (B, Hkv):
        return Hkv * n, n
    if shape == (B,) and B != Hkv:
        return n, 0
    if shape == (Hkv,) and B != Hkv:
        return 0, n
    raise ValueError(f"sigmas must be [n], [B, n], [Hkv, n] or [B, Hkv, n] (B = Hkv needs the "
                     f"3-D form); got {tuple(sigmas.shape)}")


def sa_forward_ex(q, k, v, sigmas, window: int, causal: bool, gate=None, out=None):
    """SA forward with one sigma per batch row and/or KV head (ssw_sa_forward_ex)."""
    out = _prep(q, k, v, out)
    B, n, Hq, d = q.shape
    sb, sh = _sigma_strides(sigmas, B, n, k.shape[2], q.device)
    gate = _prep_gate(gate, (B, n, Hq), q.device)
    _check(_lib.ssw_sa_forward_ex(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sigmas), sb, sh,
                                  int(window), int(bool(causal)), _dev_ptr(gate), _dev_ptr(out),
                                  B, n, Hq, k.shape[2], d, _dtype_code(q), _stream_handle(q)))
    return out


def gated_sa_swa_forward_ex(q, k, v, sigmas, window: int, causal: bool, gates, out=None):
    """Gated SA+SWA forward with one sigma per batch row and/or KV head."""
    out = _prep(q, k, v, out)
    B, n, Hq, d = q.shape
    sb, sh = _sigma_strides(sigmas, B, n, k.shape[2], q.device)
    if gates is None:
        raise ValueError("gates are required")
    gates = _prep_gate(gates, (2, B, n, Hq), q.device)
    _check(_lib.ssw_gated_sa_swa_forward_ex(_dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(sigmas),
                                            sb, sh, int(window), int(bool(causal)), _dev_ptr(gates),
                                            _dev_ptr(out), B, n, Hq, k.shape[2], d, _dtype_code(q),
                                            _stream_handle(q)))
    return out


# ------------------------------------------------------------------------------------------
# gate projections
# ------------------------------------------------------------------------------------------

def gate_projection(x, w_t, bias=None, out=None):
    """gates [2, *x.shape[:-1], Hq] = sigmoid(x @ w_t.T + bias) (ssw_gate_projection).

    x: bf16 [..., Hm] (e.g. [B, n, Hm]); w_t: bf16 [2 Hq, Hm]; bias: float32 [2 Hq] or None.
    """
    torch = _torch()
    for name, t in (("x", x), ("w_t", w_t)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous device tensor")
    if w_t.dim() != 2 or w_t.shape[1] != x.shape[-1] or w_t.shape[0] % 2:
        raise ValueError("w_t must be [2 * Hq, Hm] with Hm = x.shape[-1]")
    Hq = w_t.shape[0] // 2
    lead = tuple(x.shape[:-1])
    rows = int(np.prod(lead)) if lead else 1
    if bias is not None and (bias.dtype != torch.float32 or tuple(bias.shape) != (2 * Hq,) or
                             not bias.is_contiguous() or bias.device != x.device):
        raise ValueError("bias must be a contiguous float32 [2 * Hq] tensor on x's device")
    if out is None:
        out = torch.empty((2, *lead, Hq), dtype=torch.float32, device=x.device)
    else:
        out = _prep_rows(out, (2, *lead, Hq), torch.float32, x.device, "out")
    if x.dtype != torch.bfloat16 or w_t.dtype != torch.bfloat16:
        raise TypeError("x and w_t must be bfloat16")
    _check(_lib.ssw_gate_projection(_dev_ptr(x), _dev_ptr(w_t), _dev_ptr(bias), _dev_ptr(out),
                                    rows, x.shape[-1], Hq, BF16, _stream_handle(x)))
    return out
