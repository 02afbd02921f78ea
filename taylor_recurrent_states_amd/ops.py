"""ctypes binding of libtaylor_states.so (include/taylor_states.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory and the stream.
The calls keep the C names:

    tt_state_rows, tt_state_floats, tt_prefill_workspace_bytes, tt_prefill_workspace_bytes_dtype,
    tt_prefill, tt_prefill_from, tt_decode_step, tt_state_merge,
    tt_feature_map, tt_last_error, tt_normalize_rows,
    tt_prefill_normed_workspace_bytes, tt_prefill_normed, tt_decode_step_normed,
    tt_softmax_prefill, tt_softmax_decode_workspace_bytes, tt_softmax_decode_step,
    tt_prefill_noalloc

Loading fails loudly (ImportError / OSError) when the library has not been
built; there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree library; TT_LIBRARY names another build of the same library
# (the host-sanitizer build that the ABI tests also run against).
LIB_PATH = os.environ.get("TT_LIBRARY") or os.path.join(_PKG, "libtaylor_states.so")

TT_F32, TT_BF16 = 0, 1
TT_OK, TT_ERR_INVALID_ARG, TT_ERR_UNSUPPORTED, TT_ERR_WORKSPACE, TT_ERR_HIP = 0, -1, -2, -3, -4

EXPORTED = ("tt_state_rows", "tt_state_floats", "tt_prefill_workspace_bytes", "tt_prefill_workspace_bytes_dtype",
            "tt_prefill", "tt_prefill_from", "tt_prefill_from_unnormalized", "tt_decode_step", "tt_state_merge",
            "tt_feature_map", "tt_last_error",
            "tt_normalize_rows", "tt_prefill_normed_workspace_bytes", "tt_prefill_normed",
            "tt_decode_step_normed", "tt_softmax_prefill", "tt_softmax_decode_workspace_bytes",
            "tt_softmax_decode_step", "tt_prefill_noalloc")

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
    L.tt_prefill_workspace_bytes_dtype.argtypes = [c_int] * 8 + [ctypes.POINTER(c_size)]
    L.tt_prefill_workspace_bytes_dtype.restype = c_int
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
    L.tt_prefill_noalloc.argtypes = [c_void, c_void, c_void, c_int] + [c_int] * 7 + [c_float_p, c_float_p, c_void]
    L.tt_prefill_noalloc.restype = c_int
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
# torch plumbing.  The C entry points take raw pointers and no buffer sizes,
# so every caller-supplied buffer is checked here (dtype, element count,
# shape, contiguity, device) before the library is called: a wrong size
# would otherwise become an out-of-bounds device access.
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
    raise ValueError(f"unsupported input dtype {t.dtype} (float32 or bfloat16)")


def _contig(t, name: str):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _on_gpu(ref, *named):
    """Every tensor on the GPU, on the device of ``ref`` (checked after the
    dtypes and sizes, so that those errors do not need a GPU)."""
    for t, name in ((ref, "input"),) + named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, the inputs on {ref.device}")


def _f32(t, name: str, numel: int):
    """A caller-supplied float32 buffer of exactly ``numel`` elements."""
    torch = _torch()
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} float32 values, got {t.numel()}")
    return _contig(t, name)


class _Launch:
    """The stream of one call, and the tensors allocated for it.

    Tensors allocated here come from torch's caching allocator on the
    current stream; when the caller passes another stream they are marked
    as used on it (record_stream), so that the allocator does not hand their
    memory to a later allocation while the kernels may still run."""

    def __init__(self, stream):
        self.stream = stream
        self._resolved = None

    def _resolve(self):
        if self._resolved is None:
            torch = _torch()
            cur = torch.cuda.current_stream().cuda_stream
            s = self.stream
            if s is None:
                self._resolved = (cur, None)
            else:
                obj = s if isinstance(s, torch.cuda.Stream) else torch.cuda.ExternalStream(
                    int(getattr(s, "cuda_stream", s)))
                self._resolved = (obj.cuda_stream, obj if obj.cuda_stream != cur else None)
        return self._resolved

    @property
    def handle(self) -> int:
        return self._resolve()[0]

    def alloc(self, shape, dtype, device):
        t = _torch().empty(shape, dtype=dtype, device=device)
        other = self._resolve()[1]
        if other is not None:
            t.record_stream(other)
        return t


def _qkv(Q, K, V):
    """Shapes of prefill inputs Q, K [B, H, N, dk] and V [B, H, N, dv] of one dtype."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V")):
        if t.dim() != 4:
            raise ValueError(f"{nm} must be 4-D [B, H, N, d], got shape {tuple(t.shape)}")
    _dtype_code(Q)
    if not (Q.dtype == K.dtype == V.dtype):
        raise ValueError(f"Q, K, V must share a dtype (got {Q.dtype}, {K.dtype}, {V.dtype})")
    B, H, N, dk = Q.shape
    dv = V.shape[-1]
    if tuple(K.shape) != (B, H, N, dk) or tuple(V.shape[:3]) != (B, H, N):
        raise ValueError(f"shape mismatch: Q {tuple(Q.shape)}, K {tuple(K.shape)}, V {tuple(V.shape)}")
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V")):
        _contig(t, nm)
    return B, H, N, dk, dv


def _states_in(t, Q, K, V, n):
    """Size check of carried-in states for inputs Q, K, V (None passes)."""
    if t is not None:
        B, H, _, dk, dv = _qkv(Q, K, V)
        _f32(t, "states_in", B * H * tt_state_floats(dk, dv, n))
    return t


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


def tt_prefill_workspace_bytes_dtype(B: int, H: int, N: int, dk: int, dv: int, n: int, chunk: int = 64,
                                     dtype: str = "bf16") -> int:
    """The exact workspace of tt_prefill / tt_prefill_from for one input
    dtype ("f32" or "bf16")."""
    codes = {"f32": 0, "bf16": 1}
    if dtype not in codes:
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    out = ctypes.c_size_t(0)
    _check(lib().tt_prefill_workspace_bytes_dtype(B, H, N, dk, dv, n, chunk, codes[dtype], ctypes.byref(out)))
    return int(out.value)


def tt_prefill_normed_workspace_bytes(B: int, H: int, N: int, dk: int, dv: int, n: int, chunk: int = 64) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().tt_prefill_normed_workspace_bytes(B, H, N, dk, dv, n, chunk, ctypes.byref(out)))
    return int(out.value)


def _prefill_args(Q, K, V, n, chunk, O, states, workspace, launch, normed=False, extra=(), max_ws=None):
    torch = _torch()
    B, H, N, dk, dv = _qkv(Q, K, V)
    nstate = B * H * tt_state_floats(dk, dv, n)
    if O is not None:
        _f32(O, "O", B * H * N * dv)
    if states is not None:
        _f32(states, "states", nstate)
    if workspace is not None:
        _contig(workspace, "workspace")
    if normed:
        need = tt_prefill_normed_workspace_bytes(B, H, N, dk, dv, n, chunk)
    else:
        need = tt_prefill_workspace_bytes_dtype(B, H, N, dk, dv, n, chunk, "bf16" if _dtype_code(Q) == 1 else "f32")
    _on_gpu(Q, (K, "K"), (V, "V"), (O, "O"), (states, "states"), (workspace, "workspace"), *extra)
    if O is None:
        O = launch.alloc((B, H, N, dv), torch.float32, Q.device)
    if states is None:
        states = launch.alloc((nstate,), torch.float32, Q.device)
    if workspace is None and need > 0:
        # capped: plans that run heads in groups take a smaller workspace, the
        # library refuses it for the others (TT_ERR_WORKSPACE)
        if max_ws is not None and int(max_ws) < need:
            if int(max_ws) < 1:
                raise ValueError("max_workspace_bytes must be >= 1")
            need = int(max_ws)
        workspace = launch.alloc((need,), torch.uint8, Q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    # the caller holds ``workspace`` until the launch is queued: a workspace
    # allocated here must not return to torch's pool before that, or the next
    # allocation (an output buffer) could be handed the same memory
    return (B, H, N, dk, dv), O, states, workspace, ws_ptr, ws_bytes


def tt_prefill(Q, K, V, n: int, chunk: int = 64, O=None, states=None, workspace=None, stream=None,
               max_workspace_bytes=None):
    """Causal prefill of Q, K [B, H, N, dk] and V [B, H, N, dv] (float32 or
    bfloat16, same dtype).  Returns (O [B, H, N, dv] float32, states flat
    float32 in the library's plane layout).  Without ``workspace`` one is
    allocated for the call; ``max_workspace_bytes`` caps it, and plans with
    spans of a fixed length then run the heads in groups that fit (the
    other plans refuse a capped workspace with TT_ERR_WORKSPACE).  The same
    holds for tt_prefill_from, tt_prefill_from_unnormalized and
    tt_prefill_normed."""
    launch = _Launch(stream)
    (B, H, N, dk, dv), O, states, ws, ws_ptr, ws_bytes = _prefill_args(Q, K, V, n, chunk, O, states, workspace,
                                                                       launch, max_ws=max_workspace_bytes)
    _check(lib().tt_prefill(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk, dv, n, chunk,
                            O.data_ptr(), states.data_ptr(), ws_ptr, ws_bytes, launch.handle))
    return O, states


TT_NOALLOC_SCRATCH_BYTES = 64 << 20


def tt_prefill_noalloc(Q, K, V, n: int, chunk: int, O, states, stream=None):
    """tt_prefill that allocates nothing: O [B, H, N, dv] and states (flat,
    B*H*W*(dv+1)) float32 are required, and the library's fixed device
    scratch array serves as the workspace.  Calls that overlap on one GPU
    race.  Returns (O, states)."""
    if O is None or states is None:
        raise ValueError("tt_prefill_noalloc allocates nothing: pass O and states")
    launch = _Launch(stream)
    B, H, N, dk, dv = _qkv(Q, K, V)
    _f32(O, "O", B * H * N * dv)
    _f32(states, "states", B * H * tt_state_floats(dk, dv, n))
    _on_gpu(Q, (K, "K"), (V, "V"), (O, "O"), (states, "states"))
    _check(lib().tt_prefill_noalloc(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk, dv, n,
                                    chunk, O.data_ptr(), states.data_ptr(), launch.handle))
    return O, states


def tt_prefill_from(Q, K, V, states_in, n: int, chunk: int = 64, O=None, states=None, workspace=None,
                    stream=None, max_workspace_bytes=None):
    """Prefill continuing from carried-in states (flat float32, plane layout).
    ``states`` may be ``states_in`` itself to continue in place.  Returns
    (O, states)."""
    launch = _Launch(stream)
    if states_in is None:
        raise ValueError("states_in is None (use tt_prefill for zero states)")
    _states_in(states_in, Q, K, V, n)
    (B, H, N, dk, dv), O, states, ws, ws_ptr, ws_bytes = _prefill_args(Q, K, V, n, chunk, O, states, workspace,
                                                                       launch, extra=((states_in, "states_in"),),
                                                                       max_ws=max_workspace_bytes)
    _check(lib().tt_prefill_from(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk, dv, n,
                                 chunk, states_in.data_ptr(), O.data_ptr(), states.data_ptr(), ws_ptr, ws_bytes,
                                 launch.handle))
    return O, states


def tt_prefill_from_unnormalized(Q, K, V, states_in, n: int, chunk: int = 64, num=None, den=None, states=None,
                                 workspace=None, stream=None, max_workspace_bytes=None):
    """tt_prefill_from without the division: returns (num [B, H, N, dv],
    den [B, H, N], states); o = num / den[..., None].  ``states_in`` may be
    None (zero states)."""
    torch = _torch()
    launch = _Launch(stream)
    _states_in(states_in, Q, K, V, n)
    if den is not None:
        B, H, N, _, _ = _qkv(Q, K, V)
        _f32(den, "den", B * H * N)
    (B, H, N, dk, dv), num, states, ws, ws_ptr, ws_bytes = _prefill_args(
        Q, K, V, n, chunk, num, states, workspace, launch, extra=((states_in, "states_in"), (den, "den")),
        max_ws=max_workspace_bytes)
    if den is None:
        den = launch.alloc((B, H, N), torch.float32, Q.device)
    sin = states_in.data_ptr() if states_in is not None else 0
    _check(lib().tt_prefill_from_unnormalized(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk,
                                              dv, n, chunk, sin, num.data_ptr(), den.data_ptr(), states.data_ptr(),
                                              ws_ptr, ws_bytes, launch.handle))
    return num, den, states


def tt_prefill_normed(Q, K, V, n: int, temperature: float = 1.0, states_in=None, chunk: int = 64, O=None,
                      states=None, workspace=None, stream=None, max_workspace_bytes=None):
    """Prefill on raw Q, K: the library normalises them (Q scaled by
    ``temperature``) and runs the prefill, from ``states_in`` (flat float32,
    plane layout) or from zero states when it is None.  Returns (O, states)."""
    launch = _Launch(stream)
    _states_in(states_in, Q, K, V, n)
    (B, H, N, dk, dv), O, states, ws, ws_ptr, ws_bytes = _prefill_args(Q, K, V, n, chunk, O, states, workspace,
                                                                       launch, normed=True,
                                                                       extra=((states_in, "states_in"),),
                                                                       max_ws=max_workspace_bytes)
    sin = states_in.data_ptr() if states_in is not None else None
    _check(lib().tt_prefill_normed(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk, dv, n,
                                   chunk, float(temperature), sin, O.data_ptr(), states.data_ptr(), ws_ptr, ws_bytes,
                                   launch.handle))
    return O, states


def tt_normalize_rows(x, scale: float = 1.0, out=None, stream=None):
    """x [rows, d] (float32 or bfloat16) -> r(scale * x / ||x||) in x's dtype."""
    launch = _Launch(stream)
    _dtype_code(x)
    _contig(x, "x")
    rows, d = x.reshape(-1, x.shape[-1]).shape
    if out is not None:
        if out.dtype != x.dtype or out.shape != x.shape:
            raise ValueError("out must match x in dtype and shape")
        _contig(out, "out")
    _on_gpu(x, (out, "out"))
    if out is None:
        out = launch.alloc(tuple(x.shape), x.dtype, x.device)
    _check(lib().tt_normalize_rows(x.data_ptr(), _dtype_code(x), rows, d, float(scale), out.data_ptr(),
                                   launch.handle))
    return out


def _decode_args(q, k, v, states, n, o, launch):
    """Shapes of one decode step: q, k [B, H, dk], v [B, H, dv] of one dtype,
    states of B*H heads, o [B, H, dv] float32."""
    torch = _torch()
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        if t.dim() != 3:
            raise ValueError(f"{nm} must be 3-D [B, H, d], got shape {tuple(t.shape)}")
    _dtype_code(q)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError(f"q, k, v must share a dtype (got {q.dtype}, {k.dtype}, {v.dtype})")
    B, H, dk = q.shape
    dv = v.shape[-1]
    if tuple(k.shape) != (B, H, dk) or tuple(v.shape[:2]) != (B, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    _f32(states, "states", B * H * tt_state_floats(dk, dv, n))
    if o is not None:
        _f32(o, "o", B * H * dv)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _contig(t, nm)
    _on_gpu(q, (k, "k"), (v, "v"), (states, "states"), (o, "o"))
    if o is None:
        o = launch.alloc((B, H, dv), torch.float32, q.device)
    return B, H, dk, dv, o


def tt_decode_step_normed(q, k, v, states, n: int, temperature: float = 1.0, o=None, stream=None):
    """tt_decode_step on raw q, k (normalised in the kernel, q scaled by
    ``temperature``); states updated in place; returns o [B, H, dv]."""
    launch = _Launch(stream)
    B, H, dk, dv, o = _decode_args(q, k, v, states, n, o, launch)
    _check(lib().tt_decode_step_normed(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, dk, dv, n,
                                       float(temperature), states.data_ptr(), o.data_ptr(), launch.handle))
    return o


def tt_decode_step(q, k, v, states, n: int, o=None, stream=None):
    """One token per head: q, k [B, H, dk], v [B, H, dv]; states updated in
    place; returns o [B, H, dv] float32."""
    launch = _Launch(stream)
    B, H, dk, dv, o = _decode_args(q, k, v, states, n, o, launch)
    _check(lib().tt_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, dk, dv, n,
                                states.data_ptr(), o.data_ptr(), launch.handle))
    return o


def tt_state_merge(a, b, dst=None, stream=None):
    """dst = a + b elementwise over float32 state buffers (dst may be a or b)."""
    torch = _torch()
    launch = _Launch(stream)
    _f32(a, "a", a.numel())
    _f32(b, "b", a.numel())
    if dst is not None:
        _f32(dst, "dst", a.numel())
    _on_gpu(a, (b, "b"), (dst, "dst"))
    if dst is None:
        dst = launch.alloc(tuple(a.shape), torch.float32, a.device)
    _check(lib().tt_state_merge(dst.data_ptr(), a.data_ptr(), b.data_ptr(), a.numel(), launch.handle))
    return dst


def tt_feature_map(x, n: int, weighted: bool, out=None, stream=None):
    """x [rows, dk] -> [rows, W] float32 features (mu, or phi if weighted)."""
    torch = _torch()
    launch = _Launch(stream)
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [rows, dk], got shape {tuple(x.shape)}")
    _dtype_code(x)
    rows, dk = x.shape
    W = tt_state_rows(dk, n)
    if out is not None:
        _f32(out, "out", rows * W)
    _contig(x, "x")
    _on_gpu(x, (out, "out"))
    if out is None:
        out = launch.alloc((rows, W), torch.float32, x.device)
    _check(lib().tt_feature_map(x.data_ptr(), _dtype_code(x), rows, dk, n, int(bool(weighted)), out.data_ptr(),
                                launch.handle))
    return out


# ---------------------------------------------------------------------------
# softmax baseline
# ---------------------------------------------------------------------------

def tt_softmax_prefill(Q, K, V, O=None, stream=None):
    """Causal softmax attention (no scale) of bf16 Q, K [B, H, N, dk] and
    V [B, H, N, dv]; returns O [B, H, N, dv] float32."""
    torch = _torch()
    launch = _Launch(stream)
    B, H, N, dk, dv = _qkv(Q, K, V)
    if O is not None:
        _f32(O, "O", B * H * N * dv)
    _on_gpu(Q, (K, "K"), (V, "V"), (O, "O"))
    if O is None:
        O = launch.alloc((B, H, N, dv), torch.float32, Q.device)
    _check(lib().tt_softmax_prefill(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _dtype_code(Q), B, H, N, dk, dv,
                                    O.data_ptr(), launch.handle))
    return O


def tt_softmax_decode_workspace_bytes(B: int, H: int, pos: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().tt_softmax_decode_workspace_bytes(B, H, pos, ctypes.byref(out)))
    return int(out.value)


def tt_softmax_decode_step(q, k, v, Kcache, Vcache, pos: int, o=None, workspace=None, stream=None):
    """Append (k, v) at row ``pos`` of the caches [B, H, capacity, d] and
    return the softmax readout o [B, H, dv] float32 over rows 0 .. pos."""
    torch = _torch()
    launch = _Launch(stream)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        if t.dim() != 3:
            raise ValueError(f"{nm} must be 3-D [B, H, d], got shape {tuple(t.shape)}")
    _dtype_code(q)
    if not (q.dtype == k.dtype == v.dtype == Kcache.dtype == Vcache.dtype):
        raise ValueError("q, k, v and the caches must share a dtype")
    B, H, dk = q.shape
    dv = v.shape[-1]
    if tuple(k.shape) != (B, H, dk) or tuple(v.shape[:2]) != (B, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if Kcache.dim() != 4 or Vcache.dim() != 4:
        raise ValueError("Kcache and Vcache must be 4-D [B, H, capacity, d]")
    cap = Kcache.shape[2]
    if tuple(Kcache.shape) != (B, H, cap, dk) or tuple(Vcache.shape) != (B, H, cap, dv):
        raise ValueError(f"cache shapes {tuple(Kcache.shape)}, {tuple(Vcache.shape)} do not match q, k, v")
    if o is not None:
        _f32(o, "o", B * H * dv)
    need = tt_softmax_decode_workspace_bytes(B, H, pos)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (Kcache, "Kcache"), (Vcache, "Vcache"), (workspace, "workspace")):
        if t is not None:
            _contig(t, nm)
    if workspace is not None and workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must hold {need} bytes")
    _on_gpu(q, (k, "k"), (v, "v"), (Kcache, "Kcache"), (Vcache, "Vcache"), (o, "o"), (workspace, "workspace"))
    if o is None:
        o = launch.alloc((B, H, dv), torch.float32, q.device)
    if workspace is None:
        workspace = launch.alloc((max(need, 1),), torch.uint8, q.device)
    _check(lib().tt_softmax_decode_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, H, dk, dv,
                                        Kcache.data_ptr(), Vcache.data_ptr(), pos, cap, o.data_ptr(),
                                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                        launch.handle))
    return o
