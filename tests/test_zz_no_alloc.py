"""tt_prefill_noalloc: the prefill for callers that cannot allocate device
memory, with its workspace in the library's fixed device scratch array.
Checked through the C ABI against tt_prefill (the entry point it varies),
bit for bit: the same kernels and plans run, only the workspace differs.
Two calls in a row, the second smaller, so the second runs on scratch left
over from the first.  A streamed plan whose whole workspace exceeds the
array runs its heads in groups that fit it (same results); a shape whose
workspace exceeds the array otherwise is refused before anything is
launched."""
import numpy as np
import pytest

from gpu_util import to_device
from taylor_recurrent_states_amd import ops
from taylor_recurrent_states_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _run_both(B, H, N, dk, n, dtype, seed, chunk=64):
    import torch
    q, k, v = wl.draw_qkv(seed, B, H, N, dk, 64, dtype)
    Q, K, V = to_device(q), to_device(k), to_device(v)
    O_ref, S_ref = ops.tt_prefill(Q, K, V, n, chunk)
    O = torch.full_like(O_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    ops.tt_prefill_noalloc(Q, K, V, n, chunk, O, S)
    torch.cuda.synchronize()
    assert torch.equal(O, O_ref), f"B{B} H{H} N{N} dk{dk} n{n} {dtype}: outputs differ"
    assert torch.equal(S, S_ref), f"B{B} H{H} N{N} dk{dk} n{n} {dtype}: states differ"


def test_noalloc_matches_prefill_twice_then_smaller():
    print("\n[noalloc] prefill workload shape, bf16", flush=True)
    _run_both(4, 8, 8192, 16, 3, "bf16", 31)
    print("[noalloc] smaller second call, fp32 sweep path", flush=True)
    _run_both(1, 2, 1000, 16, 5, "f32", 32)
    print("[noalloc] smaller third call, bf16 ragged", flush=True)
    _run_both(1, 3, 777, 32, 3, "bf16", 33)


def test_noalloc_runs_streamed_heads_in_groups():
    """dk 64, n 3, bf16 on 16 heads: 81 MB of span states, 5 MB per head"""
    need = ops.tt_prefill_workspace_bytes_dtype(1, 16, 8192, 64, 64, 3, 64, "bf16")
    assert need > ops.TT_NOALLOC_SCRATCH_BYTES
    print("\n[noalloc] streamed plan in head groups", flush=True)
    _run_both(1, 16, 8192, 64, 3, "bf16", 34)


def test_noalloc_replays_in_a_captured_graph():
    """Code under graph capture is what the entry point is for: a captured
    tt_prefill_noalloc (a streamed plan in two head groups, and the pipe
    kernel's plan) is replayed three times, with an eager tt_prefill_noalloc
    on other inputs (which reuses the same scratch) between the replays;
    every replay equals the eager tt_prefill bit for bit."""
    import torch
    for B, H, N, dk, n, seed in ((1, 16, 8192, 64, 3, 35), (2, 4, 3000, 16, 3, 36)):
        print(f"\n[noalloc graph] B{B} H{H} N{N} dk{dk} n{n} bf16", flush=True)
        q, k, v = wl.draw_qkv(seed, B, H, N, dk, 64, "bf16")
        Q, K, V = to_device(q), to_device(k), to_device(v)
        O_ref, S_ref = ops.tt_prefill(Q, K, V, n)
        q2, k2, v2 = wl.draw_qkv(seed + 100, 1, 2, 1500, dk, 64, "bf16")
        Q2, K2, V2 = to_device(q2), to_device(k2), to_device(v2)
        O2 = torch.empty((1, 2, 1500, 64), device="cuda")
        S2 = torch.empty(2 * ops.tt_state_floats(dk, 64, n), device="cuda")
        O = torch.empty_like(O_ref)
        S = torch.empty_like(S_ref)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up outside the capture
            ops.tt_prefill_noalloc(Q, K, V, n, 64, O, S)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            ops.tt_prefill_noalloc(Q, K, V, n, 64, O, S)
        torch.cuda.synchronize()
        for r in range(3):
            O.fill_(float("nan"))
            S.fill_(float("nan"))
            torch.cuda.synchronize()
            gr.replay()
            torch.cuda.synchronize()
            assert torch.equal(O, O_ref), f"replay {r}: outputs"
            assert torch.equal(S, S_ref), f"replay {r}: states"
            ops.tt_prefill_noalloc(Q2, K2, V2, n, 64, O2, S2)  # eager, same scratch
            torch.cuda.synchronize()
        del gr


def test_noalloc_refuses_shapes_beyond_the_scratch():
    import torch
    # the chunk-32 sweep with row-group partial outputs: 337 MiB, no head groups
    B, H, N, dk, n, chunk = 1, 16, 8192, 16, 5, 32
    need = ops.tt_prefill_workspace_bytes_dtype(B, H, N, dk, 64, n, chunk, "f32")
    assert need > ops.TT_NOALLOC_SCRATCH_BYTES
    Q = torch.zeros((B, H, N, dk), device="cuda")
    V = torch.zeros((B, H, N, 64), device="cuda")
    O = torch.zeros((B, H, N, 64), device="cuda")
    S = torch.zeros(B * H * ops.tt_state_floats(dk, 64, n), device="cuda")
    with pytest.raises(ops.TTError) as e:
        ops.tt_prefill_noalloc(Q, Q, V, n, chunk, O, S)
    assert e.value.code == ops.TT_ERR_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not O.abs().max().item()  # nothing ran
