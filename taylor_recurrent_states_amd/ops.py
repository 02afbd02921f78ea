"""ctypes binding of libtaylor_states.so (include/taylor_states.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory and the stream.
The calls keep the C names:

    tt_state_rows, tt_state_floats, tt_prefill_workspace_bytes,
    tt_prefill, tt_prefill_from, tt_decode_step, tt_state_merge,
    tt_feature_map, tt_last_error, tt_normalize_rows,
    tt_prefill_normed_workspace_bytes, tt_prefill_normed, tt_decode_step_normed,
    tt_softmax_prefill, tt_softmax_decode_workspace_bytes, tt_softmax_decode_step

Loading fails loudly (ImportError / OSError) when the library has not been
built; there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtaylor_states.so")

TT_F32, TT_BF16 = 0, 1
TT_OK, TT_ERR_INVALID_ARG, TT_ERR_UNSUPPORTED, TT_ERR_WORKSPACE, TT_ERR_HIP = 0, -1, -2, -3, -4

EXPORTED = ("tt_state_rows", "tt_state_floats", "tt_prefill_workspace_bytes", "tt_prefill",
            "tt_prefill_from", "tt_prefill_from_unnormalized", "tt_decode_step", "tt_state_merge", "tt_feature_map", "tt_last_error",
            "tt_normalize_rows", "tt_prefill_normed_workspace_bytes", "tt_prefill_normed",
            "tt_decode_step_normed", "tt_softmax_prefill", "tt_softmax_decode_workspace_bytes",
            "tt_softmax_decode_step")

_lib = None


class TTError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded library (built by taylor_recurrent_states_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run `python -m taylor_recurrent_states_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_size, c_void, c_float_p = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
    L.tt_state_rows.argtypes = [c_int, c_int]
    L.tt_state_rows.restype = c_size
    L.tt_state_floats.argtypes = [c_int, c_int, c_int]
    L.tt_state_floats.restype = c_size
    L.tt_prefill_workspace_bytes.argtypes = [c_int] * 7 + [ctypes.POINTER(c_size)]
    L.tt_prefill_workspace_bytes.restype = c_int
    L.tt_prefill.argtypes = [c_void, c_void, c_void, c_int] + [c_int] * 7 + [c_float_p, c_float_p, c_void,
                                                                              c_size, c_void]
    L.tt_prefill.restype = c_int
    L.tt_prefill_from.argtypes = [c_void, c_void, c_void, c_int] + [c_int] * 7 + [c_float_p, c_float_p, c_float_p,
                                                                                   c_void, c_size, c_void]
    L.tt_prefill_from.restype = c_int
    L.tt_prefill_from_unnormalized.argtypes = [c_void, c_void, c_void, c_int] + [c_int] * 7 + [c_float_p] * 4 + [
        c_void, c_size, c_void]
    L.tt_prefill_from_unnormalized.restype = c_int
    L.tt_decode_step.argtypes = [c_void, c_void, c_void, c_int] + [c_int] * 5 + [c_float_p, c_float_p, c_void]
    L.tt_decode_step.restype = c_int
    L.tt_state_merge.argtypes = [c_float_p, c_float_p, c_float_p, c_size, c_void]
    L.tt_state_merge.restype = c_int
    L.tt_feature_map.argtypes = [c_void, c_int, c_size, c_int, c_int, c_int, c_float_p, c_void]
    L.tt_feature_map.restype = c_int
    c_flt = ctypes.c_float
    L.tt_normalize_rows.argtypes = [c_void, c_int, c_size, c_int, c_flt, c_void, c_void]
    L.tt_normalize_rows.restype = c_int
    L.tt_prefill_normed_workspace_bytes.argtypes = [c_int] * 7 + [ctypes.POINTER(c_size)]
    L.tt_prefill_normed_workspace_bytes.restype = c_int
    L.tt_prefill_normed.argtypes = [c_void, c_void, c_void, c_int] + [c_int] * 7 + [c_flt, c_float_p, c_float_p,
                                                                                     c_float_p, c_void, c_size, c_void]
    L.tt_prefill_normed.restype = c_int
    L.tt_decode_step_normed.argtypes = [c_void, c_void, c_void, c_int] + [c_int] * 5 + [c_flt, c_float_p, c_float_p,
                                                                                         c_void]
    L.tt_decode_step_normed.restype = c_int
    L.tt_softmax_prefill.argtypes = [c_void, c_void, c_void, c_int] + [c_int] * 5 + [c_float_p, c_void]
    L.tt_softmax_prefill.restype = c_int
    L.tt_softmax_decode_workspace_bytes.argtypes = [c_int, c_int, c_int, ctypes.POINTER(c_size)]
    L.tt_softmax_decode_workspace_bytes.restype = c_int
    L.tt_softmax_decode_step.argtypes = [c_void, c_void, c_void, c_int] + [c_int] * 4 + [c_void, c_void, c_int, c_int,
                                                                                          c_float_p, c_void, c_size,
                                                                                          c_void]
    L.tt_softmax_decode_step.restype = c_int
    L.tt_last_error.argtypes = []
    L.tt_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def tt_last_error() -> str:
    return lib().tt_last_error().decode()


def _check(rc: int) -> None:
    if rc != TT_OK:
        raise TTError(rc, tt_last_error())


# ---------------------------------------------------------------------------
# torch plumbing
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TT_F32
    if t.dtype == torch.bfloat16:
        return TT_BF16
    raise TypeError(f"unsupported input dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream) -> int:
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))
    return _torch().cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def tt_state_rows(dk: int, n: int) -> int:
    return int(lib().tt_state_rows(dk, n))


def tt_state_floats(dk: int, dv: int, n: int) -> int:
    return int(lib().tt_state_floats(dk, dv, n))


def tt_prefill_workspace_bytes(B: int, H: int, N: int, dk: int, dv: int, n: int, chunk: int = 64) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().tt_prefill_workspace_bytes(B, H, N, dk, dv, n, chunk, ctypes.byref(out)))
    return int(out.value)


def tt_prefill_normed_workspace_bytes(B: int, H: int, N: int, dk: int, dv: int, n: int, chunk: int = 64) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().tt_prefill_normed_workspace_bytes(B, H, N, dk, dv, n, chunk, ctypes.byref(out)))
    return int(out.value)


def _prefill_args(Q, K, V, n, chunk, O, states, workspace, normed=False):
    torch = _torch()
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V")):
        _dev(t, nm)
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K, V must share a dtype")
    B, H, N, dk = Q.shape
    dv = V.shape[-1]
    if tuple(K.shape) != (B, H, N, dk) or tuple(V.shape[:3]) != (B, H, N):
        raise ValueError("shape mismatch between Q, K, V")
    if O is None:
        O = torch.empty((B, H, N, dv), dtype=torch.float32, device=Q.device)
    if states is None:
        states = torch.empty(B * H * tt_state_floats(dk, dv, n), dtype=torch.float32, device=Q.device)
    need = (tt_prefill_normed_workspace_bytes if normed else tt_prefill_workspace_bytes)(B, H, N, dk, dv, n, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    # the caller holds ``workspace`` until the launch is queued: a workspace
    # allocated here must not return to torch's pool before that, or the next
    # allocation (an output buffer) could be handed the same memory
    return (B, H, N, dk, dv), O, states, workspace, ws_ptr, ws_bytes


def tt_prefill(Q, K, V, n: int, chunk: int = 64, O=None, states=None, workspace=None, stream=None):
    """Causal prefill of Q, K [B, H, N, dk] and V [B, H, N, dv] (float32 or
    bfloat16, same dtype).  Returns (O [B, H, N, dv] float32, states flat
    float32 in the library's plane layout)."""
    (B, H, N, dk, dv), O, states, ws, ws_ptr, ws_bytes = _prefill_args(Q, K, V, n, chunk, O, states, workspace)
    _check(lib().tt_prefill(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk, dv, n, chunk,
                            _dev(O, "O").data_ptr(), _dev(states, "states").data_ptr(), ws_ptr, ws_bytes,
                            _stream(stream)))
    return O, states


def tt_prefill_from(Q, K, V, states_in, n: int, chunk: int = 64, O=None, states=None, workspace=None,
                    stream=None):
    """Prefill continuing from carried-in states (flat float32, plane layout).
    ``states`` may be ``states_in`` itself to continue in place.  Returns
    (O, states)."""
    _dev(states_in, "states_in")
    (B, H, N, dk, dv), O, states, ws, ws_ptr, ws_bytes = _prefill_args(Q, K, V, n, chunk, O, states, workspace)
    if states_in.dtype != _torch().float32 or states_in.numel() != B * H * tt_state_floats(dk, dv, n):
        raise ValueError("states_in must hold B*H*W*(dv+1) float32 values")
    _check(lib().tt_prefill_from(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk, dv, n,
                                 chunk, states_in.data_ptr(), _dev(O, "O").data_ptr(),
                                 _dev(states, "states").data_ptr(), ws_ptr, ws_bytes, _stream(stream)))
    return O, states


def tt_prefill_from_unnormalized(Q, K, V, states_in, n: int, chunk: int = 64, num=None, den=None, states=None,
                                 workspace=None, stream=None):
    """tt_prefill_from without the division: returns (num [B, H, N, dv],
    den [B, H, N], states); o = num / den[..., None].  ``states_in`` may be
    None (zero states)."""
    torch = _torch()
    (B, H, N, dk, dv), num, states, ws, ws_ptr, ws_bytes = _prefill_args(Q, K, V, n, chunk, num, states, workspace)
    if den is None:
        den = torch.empty((B, H, N), dtype=torch.float32, device=Q.device)
    sin = 0
    if states_in is not None:
        _dev(states_in, "states_in")
        if states_in.dtype != torch.float32 or states_in.numel() != B * H * tt_state_floats(dk, dv, n):
            raise ValueError("states_in must hold B*H*W*(dv+1) float32 values")
        sin = states_in.data_ptr()
    if den.dtype != torch.float32 or den.numel() != B * H * N:
        raise ValueError("den must hold B*H*N float32 values")
    _check(lib().tt_prefill_from_unnormalized(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk,
                                              dv, n, chunk, sin, _dev(num, "num").data_ptr(),
                                              _dev(den, "den").data_ptr(), _dev(states, "states").data_ptr(), ws_ptr,
                                              ws_bytes, _stream(stream)))
    return num, den, states


def tt_prefill_normed(Q, K, V, n: int, temperature: float = 1.0, states_in=None, chunk: int = 64, O=None,
                      states=None, workspace=None, stream=None):
    """Prefill on raw Q, K: the library normalises them (Q scaled by
    ``temperature``) and runs the prefill, from ``states_in`` (flat float32,
    plane layout) or from zero states when it is None.  Returns (O, states)."""
    (B, H, N, dk, dv), O, states, ws, ws_ptr, ws_bytes = _prefill_args(Q, K, V, n, chunk, O, states, workspace,
                                                                   normed=True)
    sin = None
    if states_in is not None:
        _dev(states_in, "states_in")
        if states_in.dtype != _torch().float32 or states_in.numel() != B * H * tt_state_floats(dk, dv, n):
            raise ValueError("states_in must hold B*H*W*(dv+1) float32 values")
        sin = states_in.data_ptr()
    _check(lib().tt_prefill_normed(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk, dv, n,
                                   chunk, float(temperature), sin, _dev(O, "O").data_ptr(),
                                   _dev(states, "states").data_ptr(), ws_ptr, ws_bytes, _stream(stream)))
    return O, states


def tt_normalize_rows(x, scale: float = 1.0, out=None, stream=None):
    """x [rows, d] (float32 or bfloat16) -> r(scale * x / ||x||) in x's dtype."""
    torch = _torch()
    _dev(x, "x")
    rows, d = x.reshape(-1, x.shape[-1]).shape
    if out is None:
        out = torch.empty_like(x)
    if out.dtype != x.dtype or out.shape != x.shape:
        raise ValueError("out must match x in dtype and shape")
    _check(lib().tt_normalize_rows(x.data_ptr(), _dtype_code(x), rows, d, float(scale), _dev(out, "out").data_ptr(),
                                   _stream(stream)))
    return out


def tt_decode_step_normed(q, k, v, states, n: int, temperature: float = 1.0, o=None, stream=None):
    """tt_decode_step on raw q, k (normalised in the kernel, q scaled by
    ``temperature``); states updated in place; returns o [B, H, dv]."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (states, "states")):
        _dev(t, nm)
    B, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    _check(lib().tt_decode_step_normed(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, dk, dv, n,
                                       float(temperature), states.data_ptr(), _dev(o, "o").data_ptr(),
                                       _stream(stream)))
    return o


def tt_decode_step(q, k, v, states, n: int, o=None, stream=None):
    """One token per head: q, k [B, H, dk], v [B, H, dv]; states updated in
    place; returns o [B, H, dv] float32."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (states, "states")):
        _dev(t, nm)
    B, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    _check(lib().tt_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, dk, dv, n,
                                states.data_ptr(), _dev(o, "o").data_ptr(), _stream(stream)))
    return o


def tt_state_merge(a, b, dst=None, stream=None):
    """dst = a + b elementwise over float32 state buffers (dst may be a or b)."""
    torch = _torch()
    _dev(a, "a"), _dev(b, "b")
    if a.numel() != b.numel():
        raise ValueError("state buffers differ in size")
    if dst is None:
        dst = torch.empty_like(a)
    _check(lib().tt_state_merge(_dev(dst, "dst").data_ptr(), a.data_ptr(), b.data_ptr(), a.numel(),
                                _stream(stream)))
    return dst


def tt_feature_map(x, n: int, weighted: bool, out=None, stream=None):
    """x [rows, dk] -> [rows, W] float32 features (mu, or phi if weighted)."""
    torch = _torch()
    _dev(x, "x")
    rows, dk = x.shape
    W = tt_state_rows(dk, n)
    if out is None:
        out = torch.empty((rows, W), dtype=torch.float32, device=x.device)
    _check(lib().tt_feature_map(x.data_ptr(), _dtype_code(x), rows, dk, n, int(bool(weighted)),
                                _dev(out, "out").data_ptr(), _stream(stream)))
    return out


# ---------------------------------------------------------------------------
# softmax baseline
# ---------------------------------------------------------------------------

def tt_softmax_prefill(Q, K, V, O=None, stream=None):
    """Causal softmax attention (no scale) of bf16 Q, K [B, H, N, dk] and
    V [B, H, N, dv]; returns O [B, H, N, dv] float32."""
    torch = _torch()
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V")):
        _dev(t, nm)
    B, H, N, dk = Q.shape
    dv = V.shape[-1]
    if O is None:
        O = torch.empty((B, H, N, dv), dtype=torch.float32, device=Q.device)
    _check(lib().tt_softmax_prefill(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk, dv,
                                    _dev(O, "O").data_ptr(), _stream(stream)))
    return O


def tt_softmax_decode_workspace_bytes(B: int, H: int, pos: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().tt_softmax_decode_workspace_bytes(B, H, pos, ctypes.byref(out)))
    return int(out.value)


def tt_softmax_decode_step(q, k, v, Kcache, Vcache, pos: int, o=None, workspace=None, stream=None):
    """Append (k, v) at row ``pos`` of the caches [B, H, capacity, d] and
    return the softmax readout o [B, H, dv] float32 over rows 0 .. pos."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (Kcache, "Kcache"), (Vcache, "Vcache")):
        _dev(t, nm)
    B, H, dk = q.shape
    dv = v.shape[-1]
    cap = Kcache.shape[2]
    if tuple(Vcache.shape[:3]) != (B, H, cap):
        raise ValueError("Kcache and Vcache disagree in shape")
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=q.device)
    need = tt_softmax_decode_workspace_bytes(B, H, pos)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().tt_softmax_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, dk, dv,
                                        Kcache.data_ptr(), Vcache.data_ptr(), pos, cap, _dev(o, "o").data_ptr(),
                                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                        _stream(stream)))
    return o
