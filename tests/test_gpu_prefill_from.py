"""GPU parity of tt_prefill_from (prefill continued from carried-in states)
against the fp64 oracle.

The carried-in states are the oracle's states of a seeded prefix, rounded to
fp32 (the library's state dtype); the oracle continues from the same fp32
values.  Bar as for tt_prefill: fp32 inputs 1e-5 relative, bf16 inputs 5e-3
absolute.
"""
import numpy as np
import pytest

import oracle.taylor_oracle as orc
from gpu_util import assert_out, assert_states, to_device
from taylor_recurrent_states_amd import ops
from taylor_recurrent_states_amd import workloads as wl

pytestmark = pytest.mark.gpu

SHAPES = [(16, 1), (16, 2), (16, 3), (16, 4), (16, 5), (32, 1), (32, 2), (32, 3), (64, 1), (64, 2), (64, 3)]


def _tol(dtype):
    return ("rel", 1e-5) if dtype == "f32" else ("abs", 5e-3)


def _prefix_states(seed, B, H, P, dk, dv, n, dtype):
    """fp32-rounded oracle states of a seeded P-token prefix: (logical fp64
    view of the fp32 values [B, H, W, dv+1], flat device buffer)."""
    import torch
    _, k, v = wl.draw_qkv(seed, B, H, P, dk, dv, dtype)
    S = orc.states_definition(k.exact, v.exact, n).astype(np.float32).astype(np.float64)
    flat = torch.from_numpy(orc.states_to_planes(S).astype(np.float32)).cuda()
    return S, flat


@pytest.mark.parametrize("dk,n", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_from_small(dk, n, dtype):
    import torch
    B, H, P, N = 1, 2, 150, 200  # new tokens: three full chunks and a ragged tail
    S0, S0d = _prefix_states(3000 + dk * 10 + n, B, H, P, dk, 64, n, dtype)
    q, k, v = wl.draw_qkv(3100 + dk * 10 + n, B, H, N, dk, 64, dtype)
    O, S = ops.tt_prefill_from(to_device(q), to_device(k), to_device(v), S0d, n)
    torch.cuda.synchronize()
    o_ref, S_ref = orc.prefill_from_states(q.exact, k.exact, v.exact, S0, n)
    assert_out(O.cpu().numpy(), o_ref, _tol(dtype), f"dk{dk} n{n}")
    assert_states(S.cpu().numpy(), S_ref, dk, n, _tol(dtype), f"dk{dk} n{n}")
    assert torch.equal(S0d, torch.from_numpy(orc.states_to_planes(S0).astype(np.float32)).cuda())  # read-only


@pytest.mark.parametrize("N", [1, 63, 65, 300])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_from_in_place_continues_a_prefill(N, dtype):
    """tt_prefill over the first tokens, then tt_prefill_from over the rest
    with states_in == states: outputs of the second part and the final
    states equal the quadratic form and the states of the whole sequence."""
    import torch
    B, H, N1, dk, n = 2, 3, 257, 16, 3
    q, k, v = wl.draw_qkv(3200 + N, B, H, N1 + N, dk, 64, dtype)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    _, S = ops.tt_prefill(Qd[:, :, :N1].contiguous(), Kd[:, :, :N1].contiguous(), Vd[:, :, :N1].contiguous(), n)
    O2, S2 = ops.tt_prefill_from(Qd[:, :, N1:].contiguous(), Kd[:, :, N1:].contiguous(),
                                 Vd[:, :, N1:].contiguous(), S, n, states=S)
    torch.cuda.synchronize()
    assert S2.data_ptr() == S.data_ptr()
    ref = orc.quadratic_attention(q.exact, k.exact, v.exact, n)[:, :, N1:]
    assert_out(O2.cpu().numpy(), ref, _tol(dtype), f"N{N}")
    assert_states(S.cpu().numpy(), orc.states_definition(k.exact, v.exact, n), dk, n, _tol(dtype), f"N{N}")


def test_prefill_from_zero_states_equals_prefill():
    import torch
    B, H, N, dk, n = 1, 4, 333, 32, 3
    q, k, v = wl.draw_qkv(3300, B, H, N, dk, 64, "bf16")
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    Z = torch.zeros(B * H * ops.tt_state_floats(dk, 64, n), dtype=torch.float32, device="cuda")
    O1, S1 = ops.tt_prefill(Qd, Kd, Vd, n)
    O2, S2 = ops.tt_prefill_from(Qd, Kd, Vd, Z, n)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)


def test_prefill_from_workload_full_size():
    """The prefill workload (B=4, H=8, N=8192, dk=16, n=3, bf16) continued from
    the states of a 1024-token prefix per head: every state element and
    sampled output rows of every head."""
    import torch
    w = wl.WORKLOADS["prefill"]
    print("\n[prefill_from] oracle prefix states", flush=True)
    S0, S0d = _prefix_states(w.seed + 100, w.B, w.H, 1024, w.dk, w.dv, w.n, w.dtype)
    q, k, v = wl.draw_qkv(w.seed, w.B, w.H, w.N, w.dk, w.dv, w.dtype)
    O, S = ops.tt_prefill_from(to_device(q), to_device(k), to_device(v), S0d, w.n)
    torch.cuda.synchronize()
    print("[prefill_from] GPU call done", flush=True)
    BH = w.B * w.H
    Qx, Kx, Vx = (a.exact.reshape(BH, w.N, -1) for a in (q, k, v))
    S0h = S0.reshape(BH, *S0.shape[-2:])
    Og = O.cpu().numpy().reshape(BH, w.N, w.dv)
    rng = np.random.Generator(np.random.PCG64([w.seed, 98]))
    worst = 0.0
    for h in range(BH):
        rows = sorted({0, 1, 63, 64, 65, w.N // 2, w.N - 1} | set(int(x) for x in rng.integers(0, w.N, 16)))
        ref = orc.prefill_from_rows(Qx[h, rows], Kx[h], Vx[h], S0h[h], rows, w.n)
        worst = max(worst, assert_out(Og[h, rows], ref, w.tol, f"head {h}"))
    print(f"[prefill_from] sampled rows ok (worst {worst:.2e})", flush=True)
    S_ref = np.stack([orc.merge_states(S0h[h], orc.states_definition(Kx[h], Vx[h], w.n)) for h in range(BH)])
    assert_states(S.cpu().numpy(), S_ref, w.dk, w.n, w.tol, "prefill_from")
    print("[prefill_from] states ok", flush=True)


def _rel_to_max(x, ref):
    return float(np.max(np.abs(x - ref)) / max(1e-300, np.max(np.abs(ref))))


@pytest.mark.parametrize("dk,n", [(16, 2), (16, 3), (32, 2), (64, 2), (64, 3), (16, 5), (32, 4), (64, 4)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("carried", [True, False])
def test_prefill_from_unnormalized(dk, n, dtype, carried):
    """tt_prefill_from_unnormalized: the numerators and normalisers against
    the oracle's (relative to their largest element: 1e-5 for fp32 inputs,
    5e-3 for bf16), num / den at the output bar, the same states as the
    normalised call, and the normalised call's O equal to num * (1/den)
    within the hardware reciprocal's rounding.  The shapes cover the pipe
    kernel, the sweep kernel and both streamed paths (dk 64 n 3 in bf16;
    dk 16 n 5 and the run-time row tables of dk 32 and 64 with n 4)."""
    import torch
    B, H, P, N = 1, 2, 150, 200
    S0, S0d = _prefix_states(3400 + dk * 10 + n, B, H, P, dk, 64, n, dtype) if carried else (None, None)
    q, k, v = wl.draw_qkv(3500 + dk * 10 + n, B, H, N, dk, 64, dtype)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    num, den, S = ops.tt_prefill_from_unnormalized(Qd, Kd, Vd, S0d, n)
    if carried:
        O, S_n = ops.tt_prefill_from(Qd, Kd, Vd, S0d, n)
    else:
        O, S_n = ops.tt_prefill(Qd, Kd, Vd, n)
    torch.cuda.synchronize()
    num_ref, den_ref, S_ref = orc.prefill_from_numden(q.exact, k.exact, v.exact, S0, n)
    bar = 1e-5 if dtype == "f32" else 5e-3
    num_g, den_g = num.cpu().numpy().astype(np.float64), den.cpu().numpy().astype(np.float64)
    assert _rel_to_max(num_g, num_ref) <= bar, f"num dk{dk} n{n}"
    assert _rel_to_max(den_g, den_ref) <= bar, f"den dk{dk} n{n}"
    assert_out(num_g / den_g[..., None], num_ref / den_ref[..., None], _tol(dtype), f"num/den dk{dk} n{n}")
    assert_states(S.cpu().numpy(), S_ref, dk, n, _tol(dtype), f"dk{dk} n{n}")
    assert torch.equal(S, S_n)
    assert _rel_to_max(O.cpu().numpy().astype(np.float64), num_g / den_g[..., None]) <= 1e-6
