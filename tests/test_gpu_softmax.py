"""GPU parity of the softmax baseline (exact causal softmax attention, no
scale) against the fp64 oracle's softmax.

Bar: 5e-3 absolute, as for the method's bf16-input paths (the prefill feeds
bf16 probabilities to MFMA); the decode step with fp32 inputs and fp32
arithmetic is held to 1e-5 relative.
"""
import numpy as np
import pytest

import oracle.taylor_oracle as orc
from gpu_util import assert_out, to_device
from taylor_recurrent_states_amd import ops
from taylor_recurrent_states_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dk", [16, 32, 64])
@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 200, 333])
def test_softmax_prefill_small(dk, N):
    import torch
    B, H = 1, 3
    q, k, v = wl.draw_qkv(6000 + dk + N, B, H, N, dk, 64, "bf16")
    O = ops.tt_softmax_prefill(to_device(q), to_device(k), to_device(v))
    torch.cuda.synchronize()
    assert_out(O.cpu().numpy(), orc.softmax_attention(q.exact, k.exact, v.exact), ("abs", 5e-3), f"dk{dk} N{N}")


@pytest.mark.parametrize("norm", [2.0, 3.0])
def test_softmax_prefill_larger_scores(norm):
    """Rows of norm 2 and 3 (scores up to 4 and 9): the running maximum and
    the rescaling of earlier blocks are exercised."""
    import torch
    B, H, N, dk = 2, 2, 300, 16
    q, k, v = wl.draw_qkv(6100, B, H, N, dk, 64, "f32")
    q = wl.round_to(q.exact * norm, "bf16")
    k = wl.round_to(k.exact * norm, "bf16")
    v = wl.round_to(v.exact, "bf16")
    O = ops.tt_softmax_prefill(to_device(q), to_device(k), to_device(v))
    torch.cuda.synchronize()
    assert_out(O.cpu().numpy(), orc.softmax_attention(q.exact, k.exact, v.exact), ("abs", 5e-3), f"norm {norm}")


def test_softmax_prefill_full_size():
    """The prefill workload's shape (B4 H8 N8192 dk16 bf16): sampled rows of
    every head against the oracle's row-by-row softmax."""
    import torch
    w = wl.WORKLOADS["prefill"]
    q, k, v = wl.draw_qkv(w.seed, w.B, w.H, w.N, w.dk, w.dv, w.dtype)
    O = ops.tt_softmax_prefill(to_device(q), to_device(k), to_device(v))
    torch.cuda.synchronize()
    O = O.cpu().numpy().reshape(w.B * w.H, w.N, w.dv)
    BH = w.B * w.H
    Qx, Kx, Vx = (a.exact.reshape(BH, w.N, -1) for a in (q, k, v))
    rng = np.random.Generator(np.random.PCG64([w.seed, 97]))
    for h in range(BH):
        rows = sorted({0, 1, 63, 64, 65, 4095, w.N - 1} | set(int(r) for r in rng.integers(0, w.N, 8)))
        assert_out(O[h, rows], orc.softmax_rows(Qx[h, rows], Kx[h], Vx[h], rows), w.tol, f"head {h}")


def test_softmax_prefill_deterministic():
    import torch
    q, k, v = wl.draw_qkv(6200, 2, 3, 777, 32, 64, "bf16")
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    a = ops.tt_softmax_prefill(Qd, Kd, Vd)
    b = ops.tt_softmax_prefill(Qd, Kd, Vd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _decode_case(dtype, B, H, dk, P, steps, seed):
    """Cache holding P prefix tokens, then ``steps`` decode steps; every
    output against the oracle's softmax row of the whole sequence."""
    import torch
    cap = P + steps + 3
    q, k, v = wl.draw_qkv(seed, B, H, P + steps, dk, 64, dtype)
    Kd, Vd = to_device(k), to_device(v)
    Kc = torch.zeros((B, H, cap, dk), dtype=Kd.dtype, device=Kd.device)
    Vc = torch.zeros((B, H, cap, 64), dtype=Vd.dtype, device=Vd.device)
    Kc[:, :, :P] = Kd[:, :, :P]
    Vc[:, :, :P] = Vd[:, :, :P]
    Qd = to_device(q)
    tol = ("rel", 1e-5) if dtype == "f32" else ("abs", 5e-3)
    BH = B * H
    Qx, Kx, Vx = (a.exact.reshape(BH, P + steps, -1) for a in (q, k, v))
    for t in range(steps):
        pos = P + t
        o = ops.tt_softmax_decode_step(Qd[:, :, pos].contiguous(), Kd[:, :, pos].contiguous(),
                                       Vd[:, :, pos].contiguous(), Kc, Vc, pos)
        torch.cuda.synchronize()
        ref = np.stack([orc.softmax_rows(Qx[h, [pos]], Kx[h], Vx[h], [pos])[0] for h in range(BH)])
        assert_out(o.cpu().numpy().reshape(BH, 64), ref, tol, f"pos {pos}")
    # the cache now holds every token
    assert torch.equal(Kc[:, :, :P + steps], Kd) and torch.equal(Vc[:, :, :P + steps], Vd)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("P", [0, 1, 2046, 2047, 4096, 5000])
def test_softmax_decode_small(dtype, P):
    _decode_case(dtype, 2, 3, 16, P, 3, 6300 + P)


@pytest.mark.parametrize("dk", [32, 64])
def test_softmax_decode_wider_keys(dk):
    _decode_case("f32", 1, 2, dk, 3000, 2, 6400 + dk)


def test_softmax_decode_long_context():
    """A 65536-token cache (the decode workload's prefix length) for 2 x 4
    heads, fp32, two steps."""
    _decode_case("f32", 2, 4, 16, 65536, 2, 6500)
