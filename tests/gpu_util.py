"""Helpers for the GPU parity tests: device copies of seeded inputs and the
error measures the parity bar is written in."""
from __future__ import annotations

import os
import sys
from typing import Dict, Tuple

import numpy as np

import oracle.taylor_oracle as orc
from taylor_recurrent_states_amd import workloads as wl


def to_device(r: wl.Rounded):
    """Rounded input -> torch device tensor in its working dtype."""
    import torch
    if r.dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(r.device)).cuda()
    bits = np.ascontiguousarray(r.device).view(np.int16)
    return torch.from_numpy(bits).view(torch.bfloat16).cuda()


def max_abs(x, ref) -> float:
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(ref, np.float64))))


def rel(x, ref) -> float:
    """max |x - ref| / max |ref| over one tensor."""
    ref = np.asarray(ref, np.float64)
    return max_abs(x, ref) / float(np.max(np.abs(ref)))


def state_errors(flat_gpu, S_ref: np.ndarray, dk: int, n: int) -> Dict[str, Tuple[float, float]]:
    """Errors of a flat plane-layout state buffer against logical fp64
    states [..., W, e+1], per (m-block, plane): {name: (abs, rel)}."""
    S_ref = np.asarray(S_ref, np.float64)
    lead = S_ref.shape[:-2]
    W, e1 = S_ref.shape[-2:]
    BH = int(np.prod(lead)) if lead else 1
    got = orc.planes_to_states(np.asarray(flat_gpu, np.float64), 1, BH, W, e1 - 1)[0]
    ref = S_ref.reshape(BH, W, e1)
    out = {}
    for m, (a, b) in enumerate(orc.block_row_ranges(dk, n)):
        for plane, sl in (("num", slice(0, e1 - 1)), ("den", slice(e1 - 1, e1))):
            g, r = got[:, a:b, sl], ref[:, a:b, sl]
            scale = float(np.max(np.abs(r)))
            err = max_abs(g, r)
            out[f"m{m}.{plane}"] = (err, err / scale if scale > 0 else err)
    return out


def assert_states(flat_gpu, S_ref, dk, n, tol: Tuple[str, float], label=""):
    kind, bound = tol
    errs = state_errors(flat_gpu, S_ref, dk, n)
    idx = 0 if kind == "abs" else 1
    worst = max(errs.items(), key=lambda kv: kv[1][idx])
    assert worst[1][idx] <= bound, f"{label} states {worst[0]}: {kind} err {worst[1][idx]:.3e} > {bound}"
    return errs


def assert_out(o_gpu, o_ref, tol: Tuple[str, float], label=""):
    kind, bound = tol
    err = max_abs(o_gpu, o_ref) if kind == "abs" else rel(o_gpu, o_ref)
    assert err <= bound, f"{label} output {kind} err {err:.3e} > {bound}"
    return err


# ---------------------------------------------------------------------------
# Decode workload prefix: states of a seeded N-token prefix per (b, h),
# built by the oracle in fp64 and rounded to fp32 (the GPU's state dtype).
# ---------------------------------------------------------------------------

def _prefix_one(args):
    b, h, N, dk, dv, n = args
    k, v = wl.draw_prefix_kv(b, h, N, dk, dv)
    return orc.states_definition(k, v, n, block=4096)


def decode_prefix_states(B: int, H: int, N: int, dk: int, dv: int, n: int, distinct: int = 16) -> np.ndarray:
    """[B, H, W, dv+1] fp64 values of fp32-rounded prefix states.

    The oracle builds the states of ``distinct`` seeded N-token prefixes
    (heads (0, 0) .. (0, distinct-1)) and they are tiled over the B*H heads:
    heads are independent, so every head is still a valid state of a seeded
    N-token causal prefix, and the oracle checks all of them.
    """
    from concurrent.futures import ThreadPoolExecutor
    distinct = min(distinct, B * H)
    jobs = [(0, h, N, dk, dv, n) for h in range(distinct)]
    with ThreadPoolExecutor(max_workers=min(8, distinct)) as ex:
        res = list(ex.map(_prefix_one, jobs))
    base = np.stack(res)
    idx = np.arange(B * H) % distinct
    S = base[idx].reshape(B, H, *res[0].shape)
    return S.astype(np.float32).astype(np.float64)
