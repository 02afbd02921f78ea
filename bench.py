#!/usr/bin/env python3
"""Benchmark of the truncated-Taylor recurrent-state attention hot path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

Prints ONE JSON line.  A step is one tt_prefill call over the prefill
workload (B=4, H=8, N=8192, dk=16, dv=64, n=3, bf16 inputs, fp32 states
and outputs): totals, span scan and the state sweep.  `value` is prefill
tokens/s = B*N / (time per step).  The decode workload (B=64 x H=32 states
of a 65536-token prefix, 256 successive single-token steps) is timed in the
same run and reported under "decode" as us per step.  Inputs are resident
in HBM before the timed regions; timing uses HIP events on the stream the
kernels are launched on.  Before its warm-up steps every timed section runs
its step untimed for 50-200 ms, so the timed steps see the clocks of
sustained load.  "roofline" relates algorithmic bytes per launch
to the measured time; "cpu_baseline" times the fp64 oracle on the host on a
bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "prefill tokens/s @N=8192 + decode µs/token (B·H states); % of roofline"


def _source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "taylor_recurrent_states_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, src_hash):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except OSError:
        return None
    e = t.get(kernel_key)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get("bytes_per_launch")


def _prewarm(fn, torch, seconds=0.2):
    """Run fn untimed for about `seconds` of GPU time before the warm-up
    steps, so that the timed steps see the clocks the GPU settles at under
    sustained load (a few ms of work after idle run about 15 % slower)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def _time_events(fn, steps, torch):
    s = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(s)
    for _ in range(steps):
        fn()
    stop.record(s)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3  # seconds


def bench_prefill(args, torch, ops, wl):
    w = wl.WORKLOADS["prefill"]
    q, k, v = wl.draw_qkv(w.seed, w.B, w.H, w.N, w.dk, w.dv, w.dtype)
    dev = torch.device("cuda:0")

    def to_dev(r):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(r.device).view(np.int16)).view(torch.bfloat16).to(dev)

    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    O = torch.empty((w.B, w.H, w.N, w.dv), dtype=torch.float32, device=dev)
    S = torch.empty(w.B * w.H * ops.tt_state_floats(w.dk, w.dv, w.n), dtype=torch.float32, device=dev)
    ws = torch.empty(ops.tt_prefill_workspace_bytes_dtype(w.B, w.H, w.N, w.dk, w.dv, w.n, w.chunk, "bf16"),
                     dtype=torch.uint8, device=dev)

    def step():
        ops.tt_prefill(Q, K, V, w.n, w.chunk, O=O, states=S, workspace=ws)

    _prewarm(step, torch)
    for _ in range(args.warmup):
        step()
    t = _time_events(step, args.steps, torch)
    t_step = t / args.steps
    tokens = w.B * w.N
    head_tokens = w.B * w.H * w.N
    # algorithmic bytes per call: q, k (bf16) + v (bf16) read, O (fp32) written, final states written
    alg_bytes = head_tokens * (2 * w.dk * 2 + w.dv * 2 + w.dv * 4) + w.B * w.H * ops.tt_state_floats(w.dk, w.dv, w.n) * 4
    achieved = alg_bytes / t_step / 1e9
    alg_flops = 4.0 * ops.tt_state_rows(w.dk, w.n) * (w.dv + 1) * head_tokens
    src = _source_hash("tt_prefill.hip", "tt_prefill_kernels.hpp", "tt_prefill_stream.hpp", "tt_device.hpp")
    # the same workload continued from carried-in states (read once more)
    S_in = S.clone()

    def step_from():
        ops.tt_prefill_from(Q, K, V, S_in, w.n, w.chunk, O=O, states=S, workspace=ws)

    _prewarm(step_from, torch, 0.05)
    t_from = _time_events(step_from, args.steps, torch) / args.steps
    from_bytes = alg_bytes + S_in.numel() * 4
    # the same, returning numerators and normalisers (no division)
    den = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

    def step_unn():
        ops.tt_prefill_from_unnormalized(Q, K, V, S_in, w.n, w.chunk, num=O, den=den, states=S, workspace=ws)

    _prewarm(step_unn, torch, 0.05)
    t_unn = _time_events(step_unn, args.steps, torch) / args.steps
    unn_bytes = from_bytes + den.numel() * 4
    # the same workload on raw (not normalised) q, k: the library normalises
    # them (one pass over Q and K into the workspace), then runs the prefill
    qr, kr, _ = wl.draw_qkv(w.seed, w.B, w.H, w.N, w.dk, w.dv, w.dtype, normalise=False)
    Qr, Kr = to_dev(qr), to_dev(kr)
    ws_n = torch.empty(ops.tt_prefill_normed_workspace_bytes(w.B, w.H, w.N, w.dk, w.dv, w.n, w.chunk),
                       dtype=torch.uint8, device=dev)

    def step_normed():
        ops.tt_prefill_normed(Qr, Kr, V, w.n, 1.0, chunk=w.chunk, O=O, states=S, workspace=ws_n)

    _prewarm(step_normed, torch, 0.05)
    t_normed = _time_events(step_normed, args.steps, torch) / args.steps
    # the normalisation pass alone: Q and K rows in one launch
    QK = torch.cat([Qr.reshape(-1, w.dk), Kr.reshape(-1, w.dk)])
    QKn = torch.empty_like(QK)

    def step_norm():
        ops.tt_normalize_rows(QK, 1.0, out=QKn)

    _prewarm(step_norm, torch, 0.05)
    t_norm = _time_events(step_norm, args.steps, torch) / args.steps
    norm_bytes = 2 * QK.numel() * QK.element_size()
    return {
        "value": tokens / t_step, "t_step": t_step, "workload": w, "alg_bytes": alg_bytes,
        "prefill_from": {"ms_per_call": round(t_from * 1e3, 5), "tokens_per_s": round(tokens / t_from, 1),
                         "hbm_frac": round(from_bytes / t_from / 1e9 / HBM_PEAK_GBS, 4),
                         "alg_bytes_per_launch": from_bytes},
        "prefill_from_unnormalized": {"ms_per_call": round(t_unn * 1e3, 5), "tokens_per_s": round(tokens / t_unn, 1),
                                      "hbm_frac": round(unn_bytes / t_unn / 1e9 / HBM_PEAK_GBS, 4),
                                      "alg_bytes_per_launch": unn_bytes},
        "prefill_normed": {"ms_per_call": round(t_normed * 1e3, 5), "tokens_per_s": round(tokens / t_normed, 1),
                           "inputs": "raw Gaussian q, k (normalised by the library), temperature 1",
                           "normalize_pass": {"us_per_launch": round(t_norm * 1e6, 2),
                                              "alg_bytes_per_launch": norm_bytes,
                                              "achieved_GBs": round(norm_bytes / t_norm / 1e9, 1),
                                              "frac": round(norm_bytes / t_norm / 1e9 / HBM_PEAK_GBS, 4)}},
        "roofline": {"bound": "hbm", "kernel": "tt_prefill (span totals + span scan + state sweep)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": _traffic("prefill", src), "alg_bytes_per_launch": alg_bytes,
                     "source_hash": src,
                     # the contraction work of the same call against the bf16 MFMA peak
                     # (4 W (dv+1) flops per head-token: readout plus state update)
                     "mfma": {"alg_flops_per_launch": alg_flops,
                              "achieved_TFLOPs": round(alg_flops / t_step / 1e12, 2), "peak_TFLOPs": 2516.6,
                              "frac": round(alg_flops / t_step / 1e12 / 2516.6, 4)}},
        "inputs": (q, k, v),
    }


def bench_prefill_other(name, args, torch, ops, wl):
    """Secondary prefill workloads (order 5 fp32, wide head bf16): time per
    call and the MFMA roofline on algorithmic flops (4 W (dv+1) per head-token:
    readout plus state update), against the peak of the input dtype's MFMA."""
    w = wl.WORKLOADS[name]
    dev = torch.device("cuda:0")
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    tg = torch.Generator(device=dev)
    tg.manual_seed(w.seed)
    Q = torch.randn((w.B, w.H, w.N, w.dk), generator=tg, device=dev)
    K = torch.randn((w.B, w.H, w.N, w.dk), generator=tg, device=dev)
    Q = (Q / Q.norm(dim=-1, keepdim=True)).to(dt)
    K = (K / K.norm(dim=-1, keepdim=True)).to(dt)
    V = torch.randn((w.B, w.H, w.N, w.dv), generator=tg, device=dev).to(dt)
    O = torch.empty((w.B, w.H, w.N, w.dv), dtype=torch.float32, device=dev)
    S = torch.empty(w.B * w.H * ops.tt_state_floats(w.dk, w.dv, w.n), dtype=torch.float32, device=dev)
    ws_bytes = ops.tt_prefill_workspace_bytes_dtype(w.B, w.H, w.N, w.dk, w.dv, w.n, w.chunk, w.dtype)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        ops.tt_prefill(Q, K, V, w.n, w.chunk, O=O, states=S, workspace=ws)

    _prewarm(step, torch, 0.1)
    steps = max(2, min(args.steps, 10))
    t = _time_events(step, steps, torch) / steps
    W = ops.tt_state_rows(w.dk, w.n)
    flops = 4.0 * W * (w.dv + 1) * w.B * w.H * w.N
    peak = 157.3 if w.dtype == "f32" else 2516.6
    achieved = flops / t / 1e12
    # the same call with a workspace of at most 100 MB: plans whose workspace
    # is one share per head then run the heads in groups of that many shares
    small = None
    per_head = ws_bytes // (w.B * w.H)
    g = max(1, int(100e6 // per_head)) if per_head else w.B * w.H
    if g < w.B * w.H:
        ws_small = ws[: per_head * g]

        def step_small():
            ops.tt_prefill(Q, K, V, w.n, w.chunk, O=O, states=S, workspace=ws_small)

        _prewarm(step_small, torch, 0.05)
        t_s = _time_events(step_small, steps, torch) / steps
        small = {"workspace_bytes": per_head * g, "heads_per_group": g, "ms_per_call": round(t_s * 1e3, 4)}
    # the same call with the normalisation folded in (raw q, k; temperature 1)
    ws_n = torch.empty(ops.tt_prefill_normed_workspace_bytes(w.B, w.H, w.N, w.dk, w.dv, w.n, w.chunk),
                       dtype=torch.uint8, device=dev)
    del ws

    def step_n():
        ops.tt_prefill_normed(Q, K, V, w.n, 1.0, chunk=w.chunk, O=O, states=S, workspace=ws_n)

    _prewarm(step_n, torch, 0.05)
    t_n = _time_events(step_n, steps, torch) / steps
    src = _source_hash("tt_prefill.hip", "tt_prefill_kernels.hpp", "tt_prefill_stream.hpp", "tt_device.hpp")
    # algorithmic bytes: q, k, v in, O (fp32) out, final states out
    alg_bytes = w.B * w.H * w.N * (2 * w.dk + w.dv) * (4 if w.dtype == "f32" else 2) + w.B * w.H * w.N * w.dv * 4 \
        + w.B * w.H * ops.tt_state_floats(w.dk, w.dv, w.n) * 4
    return {"workload": w.name, "ms_per_call": round(t * 1e3, 4), "tokens_per_s": round(w.B * w.N / t, 1),
            "ms_per_call_normed": round(t_n * 1e3, 4), "workspace_bytes": ws_bytes, "workspace_le_100MB": small,
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(achieved / peak, 4), "alg_flops_per_launch": flops,
                         "alg_bytes_per_launch": alg_bytes, "traffic": _traffic(name, src), "source_hash": src}}


def bench_orders(args, torch, ops, wl):
    """The variant axis: time per call of the prefill workload's shape
    (B=4, H=8, N=8192, dv=64) for n = 1 .. 5 Taylor terms at dk=16 (bf16)
    and n = 1 .. 6 at dk=8 (fp32), of B=1, H=8, N=8192 for n = 1 .. 5 at
    dk=32 and 64 (bf16), and the largest deviation from exact
    softmax attention of the GPU outputs on a small seeded case (B=1, H=4,
    N=512).  The softmax reference is torch's causal attention with scale 1
    in fp64 on the CPU."""
    import math
    import numpy as np
    w = wl.WORKLOADS["prefill"]
    dev = torch.device("cuda:0")

    def to_dev(r):
        if r.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(r.device)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(r.device).view(np.int16)).view(torch.bfloat16).to(dev)

    rows = []
    # dk = 32 and 64 up to five terms (814,385 rows at dk = 64) on 8 heads
    # (B=1): the span states of all 32 heads at n = 5 would take 54 GB
    for dk, dtype, nmax, B, H in ((16, "bf16", 5, w.B, w.H), (8, "f32", 6, w.B, w.H), (32, "bf16", 5, 1, 8),
                                  (64, "bf16", 5, 1, 8)):
        q, k, v = wl.draw_qkv(w.seed, B, H, w.N, dk, w.dv, dtype)
        Q, K, V = to_dev(q), to_dev(k), to_dev(v)
        qs, ks, vs = wl.draw_qkv(4000, 1, 4, 512, dk, w.dv, dtype)
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a.exact, dtype=np.float64)) for a in (qs, ks, vs))
        o_soft = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=1.0).numpy()
        Qs, Ks, Vs = to_dev(qs), to_dev(ks), to_dev(vs)
        for n in range(1, nmax + 1):
            O = torch.empty((B, H, w.N, w.dv), dtype=torch.float32, device=dev)
            S = torch.empty(B * H * ops.tt_state_floats(dk, w.dv, n), dtype=torch.float32, device=dev)
            ws = torch.empty(ops.tt_prefill_workspace_bytes_dtype(B, H, w.N, dk, w.dv, n, w.chunk, dtype),
                             dtype=torch.uint8, device=dev)

            def step():
                ops.tt_prefill(Q, K, V, n, w.chunk, O=O, states=S, workspace=ws)

            _prewarm(step, torch, 0.05)
            steps = max(2, min(args.steps, 20))
            t = _time_events(step, steps, torch) / steps
            o_small, _ = ops.tt_prefill(Qs, Ks, Vs, n)
            err = float(np.max(np.abs(o_small.cpu().numpy().astype(np.float64) - o_soft)))
            W = ops.tt_state_rows(dk, n)
            flops = 4.0 * W * (w.dv + 1) * B * H * w.N
            rows.append({"dk": dk, "dtype": dtype, "n": n, "B": B, "H": H, "state_rows": W,
                         "ms_per_call": round(t * 1e3, 4), "tokens_per_s": round(B * w.N / t, 1),
                         "alg_TFLOPs": round(flops / t / 1e12, 2),
                         "max_abs_err_vs_softmax": err, "taylor_eps": math.e / math.factorial(n)})
            print(f"# dk={dk} {dtype} n={n}: {t * 1e6:.1f} us/call, max|o - softmax| = {err:.2e}", file=sys.stderr,
                  flush=True)
            del O, S, ws
    return {"workload": "prefill N8192 dv64: B4 H8 dk16 bf16 n=1..5, B4 H8 dk8 fp32 n=1..6, B1 H8 dk32 and dk64 "
                        "bf16 n=1..5",
            "softmax_check": "B1 H4 N512 (same dk and dtype), seed 4000", "orders": rows}


def _loglog_slope(xs, ys):
    import numpy as np
    lx, ly = np.log(np.asarray(xs, float)), np.log(np.asarray(ys, float))
    return float(np.polyfit(lx, ly, 1)[0])


def _crossover(ns, t_a, t_b):
    """Smallest N where t_a / t_b crosses 1, by log-log interpolation between
    neighbouring points; None if it does not cross in the measured range."""
    import math
    for i in range(len(ns) - 1):
        r0, r1 = t_a[i] / t_b[i], t_a[i + 1] / t_b[i + 1]
        if (r0 - 1) * (r1 - 1) <= 0 and r0 != r1:
            f = math.log(r0) / (math.log(r0) - math.log(r1))
            return round(math.exp(math.log(ns[i]) + f * (math.log(ns[i + 1]) - math.log(ns[i]))), 1)
    return None


def bench_compare(args, torch, ops, wl):
    """The pages' comparisons with softmax attention, on this GPU: prefill
    time against N (B=4, H=8, dk=16, dv=64, n=3, bf16) for the truncated
    kernel and for exact causal softmax, fitted exponents, the crossover and
    the ratio at N = 8192; decode time per step against the context length
    (B=64, H=32, fp32) for the recurrent state and for softmax over a KV
    cache, and the ratio at N = 65536."""
    w = wl.WORKLOADS["prefill"]
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    pre = []
    for N in (256, 512, 1024, 2048, 4096, 8192, 16384):
        Q = torch.randn((w.B, w.H, N, w.dk), generator=g, device=dev)
        K = torch.randn((w.B, w.H, N, w.dk), generator=g, device=dev)
        Q = (Q / Q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        K = (K / K.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        V = torch.randn((w.B, w.H, N, w.dv), generator=g, device=dev).to(torch.bfloat16)
        O = torch.empty((w.B, w.H, N, w.dv), dtype=torch.float32, device=dev)
        S = torch.empty(w.B * w.H * ops.tt_state_floats(w.dk, w.dv, w.n), dtype=torch.float32, device=dev)
        ws = torch.empty(ops.tt_prefill_workspace_bytes_dtype(w.B, w.H, N, w.dk, w.dv, w.n, w.chunk, "bf16"),
                         dtype=torch.uint8, device=dev)
        f_t = lambda: ops.tt_prefill(Q, K, V, w.n, w.chunk, O=O, states=S, workspace=ws)
        f_s = lambda: ops.tt_softmax_prefill(Q, K, V, O=O)
        row = {"N": N}
        for name, f in (("taylor_n3_us", f_t), ("softmax_us", f_s)):
            _prewarm(f, torch, 0.05)
            t1 = _time_events(f, 3, torch) / 3
            reps = max(3, min(200, int(0.1 / max(t1, 1e-6))))
            row[name] = round(_time_events(f, reps, torch) / reps * 1e6, 2)
        row["ratio_softmax_over_taylor"] = round(row["softmax_us"] / row["taylor_n3_us"], 2)
        flops = w.B * w.H * N * (N + 1) / 2 * 2 * (w.dk + w.dv)
        row["softmax_TFLOPs"] = round(flops / (row["softmax_us"] * 1e-6) / 1e12, 1)
        pre.append(row)
        print(f"# compare prefill N={N}: taylor {row['taylor_n3_us']} us, softmax {row['softmax_us']} us", file=sys.stderr,
              flush=True)
        del Q, K, V, O, S, ws
    ns = [r["N"] for r in pre]
    tt = [r["taylor_n3_us"] for r in pre]
    ts = [r["softmax_us"] for r in pre]
    big = [i for i, n in enumerate(ns) if n >= 1024]
    prefill = {"workload": "prefill B4 H8 dk16 dv64 bf16, N swept; truncated kernel n=3 vs exact causal softmax",
               "points": pre,
               "exponent_taylor_N1024_16384": round(_loglog_slope([ns[i] for i in big], [tt[i] for i in big]), 3),
               "exponent_softmax_N1024_16384": round(_loglog_slope([ns[i] for i in big], [ts[i] for i in big]), 3),
               "crossover_N": _crossover(ns, tt, ts),
               "ratio_at_8192": next(r["ratio_softmax_over_taylor"] for r in pre if r["N"] == 8192)}

    d = wl.WORKLOADS["decode"]
    BH = d.B * d.H
    nf = ops.tt_state_floats(d.dk, d.dv, d.n)
    states = torch.randn(BH * nf, generator=g, device=dev)
    q = torch.randn((d.B, d.H, d.dk), generator=g, device=dev)
    q = q / q.norm(dim=-1, keepdim=True)
    k = torch.randn((d.B, d.H, d.dk), generator=g, device=dev)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((d.B, d.H, d.dv), generator=g, device=dev)
    o = torch.empty((d.B, d.H, d.dv), dtype=torch.float32, device=dev)
    f_t = lambda: ops.tt_decode_step(q, k, v, states, d.n, o=o)
    _prewarm(f_t, torch, 0.05)
    t_taylor = _time_events(f_t, 100, torch) / 100
    dec = []
    capN = 65536 + 1
    Kc = torch.empty((d.B, d.H, capN, d.dk), dtype=torch.float32, device=dev)
    Vc = torch.empty((d.B, d.H, capN, d.dv), dtype=torch.float32, device=dev)
    for b0 in range(d.B):  # fill in slices: a normalised Gaussian cache
        kk = torch.randn((d.H, capN, d.dk), generator=g, device=dev)
        Kc[b0] = kk / kk.norm(dim=-1, keepdim=True)
        Vc[b0] = torch.randn((d.H, capN, d.dv), generator=g, device=dev)
    del kk
    ws = torch.empty(ops.tt_softmax_decode_workspace_bytes(d.B, d.H, capN - 1), dtype=torch.uint8, device=dev)
    for N in (1024, 4096, 16384, 65536):
        f_s = lambda: ops.tt_softmax_decode_step(q, k, v, Kc, Vc, N, o=o, workspace=ws)
        _prewarm(f_s, torch, 0.05)
        t1 = _time_events(f_s, 2, torch) / 2
        reps = max(2, min(100, int(0.1 / max(t1, 1e-6))))
        t_s = _time_events(f_s, reps, torch) / reps
        kv_bytes = BH * N * (d.dk + d.dv) * 4
        dec.append({"N": N, "softmax_us": round(t_s * 1e6, 2), "taylor_us": round(t_taylor * 1e6, 2),
                    "ratio_softmax_over_taylor": round(t_s / t_taylor, 1),
                    "softmax_kv_GBs": round(kv_bytes / t_s / 1e9, 1),
                    "softmax_hbm_frac": round(kv_bytes / t_s / 1e9 / HBM_PEAK_GBS, 3)})
        print(f"# compare decode N={N}: taylor {t_taylor * 1e6:.1f} us, softmax {t_s * 1e6:.1f} us", file=sys.stderr,
              flush=True)
    del Kc, Vc
    decode = {"workload": "decode B64 H32 dk16 dv64 fp32, one step at context N; recurrent state (n=3) vs softmax "
                          "over an fp32 KV cache",
              "points": dec,
              "exponent_softmax": round(_loglog_slope([r["N"] for r in dec], [r["softmax_us"] for r in dec]), 3),
              "ratio_at_65536": dec[-1]["ratio_softmax_over_taylor"]}
    return {"compare": {"prefill": prefill, "decode": decode,
                        "pages": {"prefill_exponents": "softmax N^2.28, states N^0.91", "crossover_N": 728,
                                  "ratio_at_8192": 20.8, "decode_us_per_token": 7.3, "decode_ratio_at_65536": 76.0,
                                  "hardware": "not stated"}}}


def bench_decode(args, torch, ops, wl):
    """States of a 65536-token prefix per (b, h), then 256 single-token steps."""
    w = wl.WORKLOADS["decode"]
    dev = torch.device("cuda:0")
    BH = w.B * w.H
    nf = ops.tt_state_floats(w.dk, w.dv, w.n)
    # prefix: k, v ~ N(0,1) from the seeded device generator, k L2-normalised,
    # states built with tt_prefill (fp32) in batches of heads
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    per = 256
    num = torch.empty(BH * ops.tt_state_rows(w.dk, w.n) * w.dv, dtype=torch.float32, device=dev)
    den = torch.empty(BH * ops.tt_state_rows(w.dk, w.n), dtype=torch.float32, device=dev)
    W = ops.tt_state_rows(w.dk, w.n)
    for h0 in range(0, BH, per):
        nh = min(per, BH - h0)
        kp = torch.randn((1, nh, w.N, w.dk), generator=g, device=dev)
        kp = kp / kp.norm(dim=-1, keepdim=True)
        vp = torch.randn((1, nh, w.N, w.dv), generator=g, device=dev)
        _, Sb = ops.tt_prefill(kp, kp, vp, w.n, 64)
        num[h0 * W * w.dv:(h0 + nh) * W * w.dv] = Sb[:nh * W * w.dv]
        den[h0 * W:(h0 + nh) * W] = Sb[nh * W * w.dv:]
        del kp, vp, Sb
    states = torch.cat([num, den])
    del num, den
    assert states.numel() == BH * nf
    # per-step inputs, resident before timing
    T = w.steps
    qs = torch.randn((T, w.B, w.H, w.dk), generator=g, device=dev)
    qs = qs / qs.norm(dim=-1, keepdim=True)
    ks = torch.randn((T, w.B, w.H, w.dk), generator=g, device=dev)
    ks = ks / ks.norm(dim=-1, keepdim=True)
    vs = torch.randn((T, w.B, w.H, w.dv), generator=g, device=dev)
    o = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    state_bytes = BH * nf * 4
    alg_bytes = 2 * state_bytes + BH * (2 * w.dk + w.dv) * 4 + BH * w.dv * 4

    def run(steps):
        for t in range(steps):
            ops.tt_decode_step(qs[t % T], ks[t % T], vs[t % T], states, w.n, o=o)

    # 1. one state set, steps back to back: the 81.5 MB state stays in the
    #    256 MB infinity cache (MALL) between steps
    _prewarm(lambda: run(8), torch)
    run(min(args.warmup * 4, T))
    t_warm = _time_events(lambda: run(T), 1, torch) / T
    # 2. steady state from HBM: R distinct state sets (R x 81.5 MB, larger
    #    than the MALL), step t on set t % R, so every step reads a state
    #    last touched R - 1 steps (>= 245 MB of traffic) earlier
    R = 5
    sets = [states] + [states.clone() for _ in range(R - 1)]

    def run_rot(steps):
        for t in range(steps):
            ops.tt_decode_step(qs[t % T], ks[t % T], vs[t % T], sets[t % R], w.n, o=o)

    _prewarm(lambda: run_rot(2 * R), torch)
    run_rot(min(args.warmup * 4, T))
    t_step = _time_events(lambda: run_rot(T), 1, torch) / T
    achieved = alg_bytes / t_step / 1e9
    # 3. the same T steps captured once as a HIP graph and replayed (no
    #    per-launch host cost); rotating sets and the single set
    graphs = {}
    for name, fn in (("rotating", run_rot), ("single", run)):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn(2 * R)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn(T)
        torch.cuda.synchronize()
        _prewarm(gr.replay, torch, 0.05)
        graphs[name] = _time_events(gr.replay, 4, torch) / (4 * T)
        del gr
    # 4. one step right after a 512 MB read that evicts the state (includes
    #    the latency of a single launch after an idle GPU)
    flush = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream()
    cold = []
    for t2 in range(8):
        torch.sum(flush)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        ops.tt_decode_step(qs[t2], ks[t2], vs[t2], states, w.n, o=o)
        e1.record(s)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) / 1e3)
    del flush, sets
    t_cold = sorted(cold)[len(cold) // 2]
    # raw q, k normalised inside the decode kernel (temperature 1)
    qr = torch.randn((T, w.B, w.H, w.dk), generator=g, device=dev)
    kr = torch.randn((T, w.B, w.H, w.dk), generator=g, device=dev)

    def run_normed(steps):
        for t in range(steps):
            ops.tt_decode_step_normed(qr[t % T], kr[t % T], vs[t % T], states, w.n, 1.0, o=o)

    _prewarm(lambda: run_normed(8), torch, 0.05)
    t_normed = _time_events(lambda: run_normed(T), 1, torch) / T
    src = _source_hash("tt_decode.hip", "tt_device.hpp")
    frac = lambda t: round(alg_bytes / t / 1e9 / HBM_PEAK_GBS, 4)
    return {
        "us_per_step": t_step * 1e6, "steps": T,
        "timing": f"{T} back-to-back steps rotating over {R} distinct state sets ({R * state_bytes / 1e6:.0f} MB, "
                  f"larger than the 256 MB MALL): steady-state HBM",
        "us_per_step_mall_warm": round(t_warm * 1e6, 3), "frac_mall_warm": frac(t_warm),
        "us_per_step_graph": round(graphs["rotating"] * 1e6, 3), "frac_graph": frac(graphs["rotating"]),
        "us_per_step_graph_mall_warm": round(graphs["single"] * 1e6, 3),
        "us_per_step_single_after_flush": round(t_cold * 1e6, 3),
        "us_per_step_normed": round(t_normed * 1e6, 3),
        "workload": w.name,
        "roofline": {"bound": "hbm", "kernel": "decode_kernel<16,3,float,false>", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "state_source": "HBM (rotating state sets)",
                     "traffic": _traffic("decode", src), "alg_bytes_per_launch": alg_bytes,
                     "source_hash": src},
    }


def cpu_baselines(pre, wl):
    """The fp64 oracle as it stands, on the host cores, on bounded samples."""
    import numpy as np
    import oracle.taylor_oracle as orc
    cores = len(os.sched_getaffinity(0))
    blas = "unknown"
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        blas_threads = max([i.get("num_threads", 1) for i in info] or [1])
        b = [i for i in info if i.get("user_api") == "blas"]
        if b:
            blas = f"{b[0].get('internal_api')} {b[0].get('version')} ({b[0].get('threading_layer')}, " \
                   f"{b[0].get('architecture')})"
    except Exception:
        blas_threads = cores
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    w = wl.WORKLOADS["prefill"]
    q, k, v = pre["inputs"]
    # prefill: the quadratic-form definition plus the states, head by head,
    # until about 10 s of host time
    t0 = time.perf_counter()
    heads = 0
    while heads < w.B * w.H and (heads == 0 or time.perf_counter() - t0 < 10.0):
        b, h = divmod(heads, w.H)
        orc.quadratic_attention(q.exact[b, h:h + 1], k.exact[b, h:h + 1], v.exact[b, h:h + 1], w.n)
        orc.states_definition(k.exact[b, h:h + 1], v.exact[b, h:h + 1], w.n)
        heads += 1
    t_all = time.perf_counter() - t0
    t_head = t_all / heads
    # tokens/s of the whole workload: one head-sequence is 1/(B*H) of the work
    pre_cpu = {"value": round(w.B * w.N / (t_head * w.B * w.H), 2), "unit": "tokens/s",
               "cores": blas_threads, "kind": "oracle", "cpu": cpu_model, "blas": blas,
               "sample": f"{heads} of {w.B * w.H} heads (N={w.N}): quadratic form + state definition, fp64, "
                         f"{t_all:.1f} s; scaled to B*H heads"}
    # decode: the oracle's decode step vectorised over all 2048 states, 2 steps
    d = wl.WORKLOADS["decode"]
    W = orc.state_rows(d.dk, d.n)
    rng = np.random.Generator(np.random.PCG64(5))
    S = rng.standard_normal((d.B, d.H, W, d.dv + 1))
    qq, kk, vv = wl.draw_decode_token(0, d.B, d.H, d.dk, d.dv)
    t0 = time.perf_counter()
    steps = 0
    while steps < d.steps and (steps < 2 or time.perf_counter() - t0 < 5.0):
        _, S = orc.decode_step(qq.exact, kk.exact, vv.exact, S, d.n)
        steps += 1
    t_dec = (time.perf_counter() - t0) / steps
    dec_cpu = {"value": round(t_dec * 1e6, 1), "unit": "us/step", "cores": blas_threads, "kind": "oracle",
               "cpu": cpu_model, "blas": blas,
               "sample": f"{steps} full decode steps over all {d.B * d.H} states, fp64 "
                         f"({t_dec * steps:.1f} s)"}
    return pre_cpu, dec_cpu, cores


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline (profiling runs)")
    ap.add_argument("--only", choices=["prefill", "decode", "others"], default=None)
    ap.add_argument("--compare", action="store_true",
                    help="print the comparison with exact softmax attention (prefill N sweep, decode vs context) "
                         "instead")
    ap.add_argument("--orders", action="store_true",
                    help="print the order sweep (dk16 n = 1..5, dk8 n = 1..6: time per call and error against "
                         "softmax) instead")
    ap.add_argument("--calibrate", action="store_true",
                    help="run only tt_state_merge over 2 x 256 MiB -> 256 MiB (known HBM bytes), "
                         "to scale the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU and the hot path has no multi-GPU code; run with --gpus 1. "
              "(Heads shard with no exchange; sequence segments would exchange one state set per GPU, "
              "because the states add.)", file=sys.stderr)
        sys.exit(2)

    import torch
    from taylor_recurrent_states_amd import ops
    from taylor_recurrent_states_amd import workloads as wl
    ops.lib()  # fails loudly if the library is not built
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.compare:
        print(json.dumps(bench_compare(args, torch, ops, wl)), flush=True)
        return

    if args.orders:
        print(json.dumps(bench_orders(args, torch, ops, wl)), flush=True)
        return

    if args.calibrate:
        n = 64 * 1024 * 1024
        a = torch.ones(n, device="cuda")
        b = torch.ones(n, device="cuda")
        d = torch.empty(n, device="cuda")
        for _ in range(3):
            ops.tt_state_merge(a, b, dst=d)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate": "tt_state_merge", "read_bytes_per_launch": 2 * n * 4,
                          "write_bytes_per_launch": n * 4, "launches": 3}), flush=True)
        return

    pre = dec = None
    if args.only in (None, "prefill"):
        pre = bench_prefill(args, torch, ops, wl)
        print(f"# prefill: {pre['t_step'] * 1e6:.1f} us/step, {pre['value']:.4g} tokens/s", file=sys.stderr,
              flush=True)
    if args.only in (None, "decode"):
        dec = bench_decode(args, torch, ops, wl)
        print(f"# decode: {dec['us_per_step']:.2f} us/step", file=sys.stderr, flush=True)
    others = {}
    if args.only in (None, "others"):
        for name in ("order5", "wide"):
            others[name] = bench_prefill_other(name, args, torch, ops, wl)
            print(f"# {name}: {others[name]['ms_per_call']:.3f} ms/call", file=sys.stderr, flush=True)

    out = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}
    w = wl.WORKLOADS["prefill"]
    if pre is not None:
        out.update({"value": round(pre["value"], 1), "ms_per_step": round(pre["t_step"] * 1e3, 5),
                    "roofline": pre["roofline"], "prefill_from": pre["prefill_from"],
                    "prefill_from_unnormalized": pre["prefill_from_unnormalized"],
                    "prefill_normed": pre["prefill_normed"]})
    else:
        out.update({"value": None, "ms_per_step": None, "roofline": None})
    out["config"] = {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "dk": w.dk, "dv": w.dv, "n": w.n,
                     "chunk": w.chunk, "states": "fp32", "outputs": "fp32",
                     "decode_workload": wl.WORKLOADS["decode"].name}
    if dec is not None:
        out["decode"] = dec
    if others:
        out["other_prefill_workloads"] = others
    if not args.no_cpu and pre is not None:
        pre_cpu, dec_cpu, cores = cpu_baselines(pre, wl)
        out["cpu_baseline"] = pre_cpu
        if dec is not None:
            out["decode"]["cpu_baseline"] = dec_cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
