"""Calls on a caller-supplied stream: the work runs on that stream, and
buffers the binding allocates for the call are not handed to another
allocation on the current stream while the kernels may still run."""
import numpy as np
import pytest

from gpu_util import to_device
from taylor_recurrent_states_amd import ops
from taylor_recurrent_states_amd import workloads as wl

pytestmark = pytest.mark.gpu


def test_prefill_on_a_side_stream():
    import torch
    B, H, N, dk, n = 2, 4, 2000, 16, 3
    q, k, v = wl.draw_qkv(9100, B, H, N, dk, 64, "bf16")
    Q, K, V = to_device(q), to_device(k), to_device(v)
    O_ref, S_ref = ops.tt_prefill(Q, K, V, n)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        O, S = ops.tt_prefill(Q, K, V, n, stream=side)  # workspace allocated by the binding
        # allocations on the current stream right after the call must not
        # reuse the workspace while the side stream may still read it
        junk = [torch.full((1 << 20,), 7.0, device="cuda") for _ in range(8)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(O, O_ref) and torch.equal(S, S_ref)
        del junk


def test_softmax_decode_on_a_side_stream():
    import torch
    B, H, dk, dv, cap, pos = 2, 4, 16, 64, 5000, 4100
    g = torch.Generator(device="cuda")
    g.manual_seed(9200)
    Kc = torch.randn((B, H, cap, dk), generator=g, device="cuda")
    Vc = torch.randn((B, H, cap, dv), generator=g, device="cuda")
    q = torch.randn((B, H, dk), generator=g, device="cuda")
    k = torch.randn((B, H, dk), generator=g, device="cuda")
    v = torch.randn((B, H, dv), generator=g, device="cuda")
    Kc2, Vc2 = Kc.clone(), Vc.clone()
    o_ref = ops.tt_softmax_decode_step(q, k, v, Kc, Vc, pos)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o = ops.tt_softmax_decode_step(q, k, v, Kc2, Vc2, pos, stream=side)
    junk = [torch.full((1 << 20,), 3.0, device="cuda") for _ in range(8)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    assert torch.equal(Kc2[:, :, pos], k) and torch.equal(Vc2[:, :, pos], v)
    del junk
