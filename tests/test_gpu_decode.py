"""GPU parity: feature map, decode step and state merge against the fp64 oracle.

Tolerances: fp32 paths 1e-5 relative (max|x - ref| / max|ref| per output
tensor; per (m-block, plane) for states), bf16-input paths 5e-3 absolute.
"""
import numpy as np
import pytest

import oracle.taylor_oracle as orc
from gpu_util import assert_out, assert_states, decode_prefix_states, to_device
from taylor_recurrent_states_amd import ops
from taylor_recurrent_states_amd import workloads as wl

pytestmark = pytest.mark.gpu

SHAPES = [(8, 3), (8, 6), (16, 1), (16, 2), (16, 3), (16, 4), (16, 5), (32, 3), (64, 2), (64, 3)]


@pytest.mark.parametrize("dk,n", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_feature_map(dk, n, dtype):
    import torch
    rows = 37
    q, _, _ = wl.draw_qkv(100 + dk + n, 1, 1, rows, dk, 4, dtype)
    x = to_device(q)[0, 0]
    for weighted in (False, True):
        got = ops.tt_feature_map(x, n, weighted).cpu().numpy()
        ref = orc.feature_map(q.exact[0, 0], n, weighted)
        assert got.shape == ref.shape
        assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref))
    torch.cuda.synchronize()


def _decode_run(B, H, dk, n, steps, dtype, prefix_N, seed):
    import torch
    dv = 64
    q0, k0, v0 = wl.draw_qkv(seed, B, H, prefix_N, dk, dv, "f32")
    S0 = orc.states_definition(k0.exact, v0.exact, n).astype(np.float32).astype(np.float64)
    states = torch.from_numpy(orc.states_to_planes(S0).astype(np.float32)).cuda()
    S = S0
    for t in range(steps):
        q, k, v = wl.draw_qkv((seed, t), B, H, 1, dk, dv, dtype)
        o = ops.tt_decode_step(to_device(q)[:, :, 0].contiguous(), to_device(k)[:, :, 0].contiguous(),
                               to_device(v)[:, :, 0].contiguous(), states, n)
        o_ref, S = orc.decode_step(q.exact[:, :, 0], k.exact[:, :, 0], v.exact[:, :, 0], S, n)
        torch.cuda.synchronize()
        tol = ("rel", 1e-5) if dtype == "f32" else ("abs", 5e-3)
        assert_out(o.cpu().numpy(), o_ref, tol, f"step {t}")
    assert_states(states.cpu().numpy(), S, dk, n, ("rel", 1e-5) if dtype == "f32" else ("abs", 5e-3))
    return states


@pytest.mark.parametrize("dk,n", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_small(dk, n, dtype):
    _decode_run(2, 3, dk, n, steps=4, dtype=dtype, prefix_N=50, seed=7)


def test_decode_from_zero_equals_quadratic():
    """N decode steps from zero states reproduce the causal quadratic form."""
    import torch
    B, H, N, dk, dv, n = 1, 2, 40, 16, 64, 3
    q, k, v = wl.draw_qkv(77, B, H, N, dk, dv, "f32")
    states = torch.zeros(B * H * ops.tt_state_floats(dk, dv, n), device="cuda")
    Q, K, V = to_device(q), to_device(k), to_device(v)
    outs = [ops.tt_decode_step(Q[:, :, t].contiguous(), K[:, :, t].contiguous(), V[:, :, t].contiguous(),
                               states, n).cpu().numpy() for t in range(N)]
    o = np.stack(outs, axis=2)
    assert_out(o, orc.quadratic_attention(q.exact, k.exact, v.exact, n), ("rel", 1e-5))
    assert_states(states.cpu().numpy(), orc.states_definition(k.exact, v.exact, n), dk, n, ("rel", 1e-5))


def test_decode_bitwise_repeatable():
    import torch
    a = _decode_run(2, 2, 16, 3, steps=3, dtype="f32", prefix_N=30, seed=9).cpu().numpy()
    b = _decode_run(2, 2, 16, 3, steps=3, dtype="f32", prefix_N=30, seed=9).cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.timeout(600)
def test_decode_full_workload_every_step():
    """The decode workload at full size (B=64, H=32, dk=16, n=3, a different
    65536-token prefix state for every head): every output of all 256 steps
    matches the oracle, and so do all states after steps 1, 64 and 256; the
    steps run in the launch configuration the bench times."""
    import torch
    w = wl.WORKLOADS["decode"]
    print("\n[decode] building prefix states", flush=True)
    S = decode_prefix_states(w.B, w.H, w.N, w.dk, w.dv, w.n)
    states = torch.from_numpy(orc.states_to_planes(S).astype(np.float32)).cuda()
    worst = 0.0
    for t in range(w.steps):
        q, k, v = wl.draw_decode_token(t, w.B, w.H, w.dk, w.dv)
        o = ops.tt_decode_step(to_device(q), to_device(k), to_device(v), states, w.n)
        o_ref, S = orc.decode_step(q.exact, k.exact, v.exact, S, w.n)
        torch.cuda.synchronize()
        worst = max(worst, assert_out(o.cpu().numpy(), o_ref, ("rel", 1e-5), f"step {t}"))
        if t + 1 in (1, 64, w.steps):
            assert_states(states.cpu().numpy(), S, w.dk, w.n, ("rel", 1e-5), f"after step {t + 1}")
            print(f"[decode] states after step {t + 1} ok; worst output error so far {worst:.2e}", flush=True)


@pytest.mark.parametrize("nfloats", [1, 3, 4, 9945, 9945 * 32 + 1])
def test_merge(nfloats):
    import torch
    g = np.random.Generator(np.random.PCG64(nfloats))
    a = g.standard_normal(nfloats).astype(np.float32)
    b = g.standard_normal(nfloats).astype(np.float32)
    A, Bt = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    out = ops.tt_state_merge(A, Bt).cpu().numpy()
    assert np.array_equal(out, a + b)
    ops.tt_state_merge(A, Bt, dst=A)  # in place, aliasing a
    assert np.array_equal(A.cpu().numpy(), a + b)
    # misaligned views take the scalar path
    if nfloats > 2:
        A2 = torch.from_numpy(a).cuda()
        got = ops.tt_state_merge(A2[1:], Bt[1:]).cpu().numpy()
        assert np.array_equal(got, a[1:] + b[1:])


def test_decode_graph_replays_match_eager():
    """Eight decode steps captured once as a HIP graph (the launch the bench
    times as its graph variant) and replayed three times, with eager work
    and synchronisation between replays: after every replay the outputs and
    the states equal those of the same steps run eagerly, bit for bit."""
    import torch
    B, H, dk, dv, n, T = 4, 8, 16, 64, 3, 8
    g = torch.Generator(device="cuda")
    g.manual_seed(9300)
    nf = ops.tt_state_floats(dk, dv, n)
    S_graph = torch.randn(B * H * nf, generator=g, device="cuda").abs()
    S_eager = S_graph.clone()
    qs = torch.nn.functional.normalize(torch.randn((T, B, H, dk), generator=g, device="cuda"), dim=-1)
    ks = torch.nn.functional.normalize(torch.randn((T, B, H, dk), generator=g, device="cuda"), dim=-1)
    vs = torch.randn((T, B, H, dv), generator=g, device="cuda")
    o_graph = torch.empty((T, B, H, dv), device="cuda")
    o_eager = torch.empty_like(o_graph)

    def steps(S, out):
        for t in range(T):
            ops.tt_decode_step(qs[t], ks[t], vs[t], S, n, o=out[t])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, on a scratch copy
        scratch = S_graph.clone()
        steps(scratch, torch.empty_like(o_graph))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        steps(S_graph, o_graph)
    torch.cuda.synchronize()
    for r in range(3):
        gr.replay()
        torch.cuda.synchronize()
        steps(S_eager, o_eager)
        _ = (scratch * 2).sum().item()  # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o_graph, o_eager), f"replay {r}: outputs"
        assert torch.equal(S_graph, S_eager), f"replay {r}: states"
