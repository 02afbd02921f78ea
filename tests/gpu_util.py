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
# Oracle work of the full-size tests, spread over CPU processes.  The oracle
# is single-threaded numpy; heads are independent, so the reference of each
# head is computed in its own process (spawned: the children import only
# numpy and the oracle, never the GPU runtime).
# ---------------------------------------------------------------------------

def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(1)
    except ImportError:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


def _states_job(args):
    K, V, n = args
    with _one_thread():
        return orc.states_definition(K, V, n, block=4096)


def _rows_job(args):
    q_rows, K, V, rows, n = args
    with _one_thread():
        return orc.quadratic_rows(q_rows, K, V, rows, n)


def _prefix_job(args):
    b, h, N, dk, dv, n, part = args
    k, v = wl.draw_prefix_kv(b, h, N, dk, dv, part)
    with _one_thread():
        return orc.states_definition(k, v, n, block=4096)


def oracle_map(fn, jobs, workers: int = 16):
    """[fn(job) for job in jobs], computed in up to ``workers`` spawned
    processes (at most 16: the CPU share of one GPU)."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    jobs = list(jobs)
    if len(jobs) <= 1:
        return [fn(j) for j in jobs]
    from concurrent.futures.process import BrokenProcessPool
    workers = max(1, min(workers, 16, len(jobs), os.cpu_count() or 1))
    try:
        with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
            return list(ex.map(fn, jobs))
    except (BrokenProcessPool, OSError) as e:  # no child processes here: the same work in this process
        print(f"[oracle] process pool unavailable ({e!r}); computing serially", flush=True)
        return [fn(j) for j in jobs]


def oracle_states(K, V, n: int, heads):
    """Oracle states of the listed heads: K [BH, N, d], V [BH, N, e] (fp64)."""
    return oracle_map(_states_job, [(K[h], V[h], n) for h in heads])


def oracle_rows(Q, K, V, rows_of, n: int, heads):
    """Oracle outputs at the sampled rows ``rows_of[h]`` of the listed heads."""
    return oracle_map(_rows_job, [(Q[h, rows_of[h]], K[h], V[h], rows_of[h], n) for h in heads])


# ---------------------------------------------------------------------------
# Decode workload prefix: states of a seeded N-token prefix per (b, h),
# built by the oracle in fp64 and rounded to fp32 (the GPU's state dtype).
# ---------------------------------------------------------------------------

def decode_prefix_states(B: int, H: int, N: int, dk: int, dv: int, n: int, distinct: int = 16,
                         tail: int = 256) -> np.ndarray:
    """[B, H, W, dv+1] fp64 values of fp32-rounded prefix states, a different
    one for every head.

    Head (b, h)'s prefix is N - ``tail`` tokens shared with every
    ``distinct``-th head (the oracle builds ``distinct`` seeded prefixes,
    PCG64([2, 0, i])) followed by ``tail`` tokens of its own
    (PCG64([2, b, h, 1])).  States add over token sets, so the sum of the two
    states is the state of that N-token causal prefix; building all B*H
    prefixes in full would take the CPU oracle hours.
    """
    distinct = min(distinct, B * H)
    base = np.stack(oracle_map(_prefix_job, [(0, i, N - tail, dk, dv, n, 0) for i in range(distinct)]))
    heads = [(b, h) for b in range(B) for h in range(H)]
    Kt = np.empty((B * H, tail, dk))
    Vt = np.empty((B * H, tail, dv))
    for i, (b, h) in enumerate(heads):
        Kt[i], Vt[i] = wl.draw_prefix_kv(b, h, tail, dk, dv, part=1)
    chunks = np.array_split(np.arange(B * H), 16)
    tails = np.concatenate(oracle_map(_states_job, [(Kt[c], Vt[c], n) for c in chunks]))
    S = base[np.arange(B * H) % distinct] + tails
    return S.reshape(B, H, *S.shape[1:]).astype(np.float32).astype(np.float64)
