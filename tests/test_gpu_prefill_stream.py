"""GPU parity of the streamed-state prefill path (bf16 inputs with n = 3 and
dk = 32 or 64; fp32 inputs with more than 256 feature rows) over several
spans: the span totals, their exclusive scan rewritten as readout fragments,
and the output pass that adds the readout of the prefix state to the span's
own causal block ("Expanding Attention", abstract: the states of disjoint
token sets add; comment thread item 46888355: (Q'K)V = Q'(KV) for everything
but the span's causal block).

Spans are 1024 tokens, so lengths above 1024 exercise the prefix readout,
the scan over several spans and the ragged last span.  The bars are 5e-3
absolute for bf16 inputs and 1e-5 relative for fp32, against the oracle's
fp64 quadratic form; for bf16, values offset from zero (v ~ N(3, 1)) and four
times wider (v ~ 4 N(0, 1)) are included, where a readout that rounded the
state to one bf16 would fail.
"""
import numpy as np
import pytest

import oracle.taylor_oracle as orc
from gpu_util import assert_out, assert_states, to_device
from taylor_recurrent_states_amd import ops
from taylor_recurrent_states_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = ("abs", 5e-3)


def _draw(seed, B, H, N, dk, shift=0.0, scale=1.0):
    q, k, v = wl.draw_qkv(seed, B, H, N, dk, 64, "bf16")
    if shift != 0.0 or scale != 1.0:
        v = wl.round_to(shift + scale * v.exact, "bf16")
    return q, k, v


@pytest.mark.parametrize("dk", [32, 64])
@pytest.mark.parametrize("N", [1025, 2048, 3001])
def test_stream_prefill_several_spans(dk, N):
    import torch
    q, k, v = _draw(5000 + dk + N, 1, 2, N, dk)
    O, S = ops.tt_prefill(to_device(q), to_device(k), to_device(v), 3)
    torch.cuda.synchronize()
    assert_out(O.cpu().numpy(), orc.quadratic_attention(q.exact, k.exact, v.exact, 3), TOL, f"dk{dk} N{N}")
    assert_states(S.cpu().numpy(), orc.states_definition(k.exact, v.exact, 3), dk, 3, TOL, f"dk{dk} N{N}")


@pytest.mark.parametrize("shift,scale", [(3.0, 1.0), (0.0, 4.0)])
def test_stream_prefill_offset_values(shift, scale):
    import torch
    dk, N = 64, 3001
    q, k, v = _draw(5100, 1, 2, N, dk, shift, scale)
    O, S = ops.tt_prefill(to_device(q), to_device(k), to_device(v), 3)
    torch.cuda.synchronize()
    assert_out(O.cpu().numpy(), orc.quadratic_attention(q.exact, k.exact, v.exact, 3), TOL, f"v~{shift}+{scale}N")
    assert_states(S.cpu().numpy(), orc.states_definition(k.exact, v.exact, 3), dk, 3, TOL, f"v~{shift}+{scale}N")


@pytest.mark.parametrize("dk", [32, 64])
def test_stream_prefill_from_states_and_unnormalized(dk):
    """Continued from carried-in states (the oracle's states of a 700-token
    prefix, rounded to fp32) over 2500 new tokens: outputs, numerators,
    normalisers and final states against the oracle."""
    import torch
    B, H, P, N = 1, 2, 700, 2500
    _, kp, vp = _draw(5200 + dk, B, H, P, dk)
    S0 = orc.states_definition(kp.exact, vp.exact, 3).astype(np.float32).astype(np.float64)
    S0d = torch.from_numpy(orc.states_to_planes(S0).astype(np.float32)).cuda()
    q, k, v = _draw(5300 + dk, B, H, N, dk)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    O, S = ops.tt_prefill_from(Qd, Kd, Vd, S0d, 3)
    num, den, S_u = ops.tt_prefill_from_unnormalized(Qd, Kd, Vd, S0d, 3)
    torch.cuda.synchronize()
    num_ref, den_ref, S_ref = orc.prefill_from_numden(q.exact, k.exact, v.exact, S0, 3)
    assert_out(O.cpu().numpy(), num_ref / den_ref[..., None], TOL, f"from dk{dk}")
    assert_states(S.cpu().numpy(), S_ref, dk, 3, TOL, f"from dk{dk}")
    num_g, den_g = num.cpu().numpy().astype(np.float64), den.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(num_g - num_ref)) <= 5e-3 * np.max(np.abs(num_ref))
    assert np.max(np.abs(den_g - den_ref)) <= 5e-3 * np.max(np.abs(den_ref))
    assert torch.equal(S, S_u)
    o_g = O.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(o_g - num_g / den_g[..., None])) <= 1e-6 * np.max(np.abs(o_g))


def test_stream_prefill_agrees_with_the_chunk_32_sweep():
    """Chunk 64 runs this path, chunk 32 the sweep kernel that carries the
    state through the span: two implementations of the same quantity."""
    import torch
    dk, N = 64, 2600
    q, k, v = _draw(5400, 1, 2, N, dk)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    O64, S64 = ops.tt_prefill(Qd, Kd, Vd, 3, 64)
    O32, S32 = ops.tt_prefill(Qd, Kd, Vd, 3, 32)
    torch.cuda.synchronize()
    assert float((O64 - O32).abs().max()) <= 5e-3
    ref = orc.states_definition(k.exact, v.exact, 3)
    assert_states(S64.cpu().numpy(), ref, dk, 3, TOL, "chunk 64")
    assert_states(S32.cpu().numpy(), ref, dk, 3, TOL, "chunk 32")


def test_stream_prefill_repeatable():
    import torch
    q, k, v = _draw(5500, 2, 2, 1500, 64)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    O1, S1 = ops.tt_prefill(Qd, Kd, Vd, 3)
    O2, S2 = ops.tt_prefill(Qd, Kd, Vd, 3)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)


# ---------------------------------------------------------------------------
# fp32 inputs with more than 256 feature rows take the same structure on fp32
# MFMA (order 5 at dk = 16, n >= 5 at dk = 8): several spans with a ragged
# last one, carried-in states and the unnormalised form.  Bar: 1e-5 relative.
# ---------------------------------------------------------------------------

F32_TOL = ("rel", 1e-5)


@pytest.mark.parametrize("dk,n,N", [(16, 5, 3001), (8, 6, 2100), (8, 5, 1025)])
def test_stream_f32_several_spans(dk, n, N):
    import torch
    q, k, v = wl.draw_qkv(5600 + 10 * dk + n, 1, 2, N, dk, 64, "f32")
    O, S = ops.tt_prefill(to_device(q), to_device(k), to_device(v), n)
    torch.cuda.synchronize()
    assert_out(O.cpu().numpy(), orc.quadratic_attention(q.exact, k.exact, v.exact, n), F32_TOL, f"dk{dk} n{n} N{N}")
    assert_states(S.cpu().numpy(), orc.states_definition(k.exact, v.exact, n), dk, n, F32_TOL, f"dk{dk} n{n} N{N}")


def test_stream_f32_from_states_and_unnormalized():
    """dk = 16, n = 5 continued from the oracle's states of a 900-token prefix
    (rounded to fp32) over 2100 new tokens."""
    import torch
    dk, n, P, N = 16, 5, 900, 2100
    _, kp, vp = wl.draw_qkv(5700, 1, 2, P, dk, 64, "f32")
    S0 = orc.states_definition(kp.exact, vp.exact, n).astype(np.float32).astype(np.float64)
    S0d = torch.from_numpy(orc.states_to_planes(S0).astype(np.float32)).cuda()
    q, k, v = wl.draw_qkv(5701, 1, 2, N, dk, 64, "f32")
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    O, S = ops.tt_prefill_from(Qd, Kd, Vd, S0d, n)
    num, den, S_u = ops.tt_prefill_from_unnormalized(Qd, Kd, Vd, S0d, n)
    torch.cuda.synchronize()
    num_ref, den_ref, S_ref = orc.prefill_from_numden(q.exact, k.exact, v.exact, S0, n)
    assert_out(O.cpu().numpy(), num_ref / den_ref[..., None], F32_TOL, "from f32")
    assert_states(S.cpu().numpy(), S_ref, dk, n, F32_TOL, "from f32")
    num_g, den_g = num.cpu().numpy().astype(np.float64), den.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(num_g - num_ref)) <= 1e-5 * np.max(np.abs(num_ref))
    assert np.max(np.abs(den_g - den_ref)) <= 1e-5 * np.max(np.abs(den_ref))
    assert torch.equal(S, S_u)
