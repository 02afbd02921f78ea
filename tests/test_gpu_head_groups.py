"""Prefill with a workspace that holds the span states of fewer heads than
the call has.  Plans whose spans have a fixed length (the streamed paths:
bf16 with n = 3 at dk = 32 and 64, fp32 with more than 256 feature rows,
four or more terms) then run the heads in groups, one after another, each
group through the same kernels and the same spans, so every output and
state must be bit-identical to the call with the whole workspace.  Checked
for tt_prefill, tt_prefill_from (carried-in states of the heads of every
group), tt_prefill_from_unnormalized and tt_prefill_normed (each group's
rows of Q and K normalised into its share of the workspace); a workspace
below one head's share is refused before anything runs."""
import pytest

from gpu_util import to_device
from taylor_recurrent_states_amd import ops
from taylor_recurrent_states_amd import workloads as wl

pytestmark = pytest.mark.gpu

# (B, H, N, dk, n, dtype, heads per group)
CASES = [(1, 5, 2100, 64, 3, "bf16", 2), (2, 2, 1500, 16, 5, "f32", 1), (1, 3, 1100, 32, 4, "bf16", 2)]


@pytest.mark.parametrize("B,H,N,dk,n,dtype,group", CASES)
def test_head_groups_match_the_whole_workspace(B, H, N, dk, n, dtype, group):
    import torch
    print(f"\n[groups] B{B} H{H} N{N} dk{dk} n{n} {dtype}, {group} heads per group", flush=True)
    q, k, v = wl.draw_qkv(5100 + dk + n, B, H, N, dk, 64, dtype)
    Q, K, V = to_device(q), to_device(k), to_device(v)
    need = ops.tt_prefill_workspace_bytes_dtype(B, H, N, dk, 64, n, 64, dtype)
    per_head = need // (B * H)
    assert per_head * B * H == need
    small = torch.empty(per_head * group + 100, dtype=torch.uint8, device="cuda")
    O_ref, S_ref = ops.tt_prefill(Q, K, V, n)
    O, S = ops.tt_prefill(Q, K, V, n, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(O, O_ref) and torch.equal(S, S_ref), "tt_prefill"
    # continued from the states of the first call (a different state per head)
    O2_ref, S2_ref = ops.tt_prefill_from(Q, K, V, S_ref, n)
    O2, S2 = ops.tt_prefill_from(Q, K, V, S_ref, n, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(O2, O2_ref) and torch.equal(S2, S2_ref), "tt_prefill_from"
    num_ref, den_ref, S3_ref = ops.tt_prefill_from_unnormalized(Q, K, V, S_ref, n)
    num, den, S3 = ops.tt_prefill_from_unnormalized(Q, K, V, S_ref, n, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(num, num_ref) and torch.equal(den, den_ref) and torch.equal(S3, S3_ref), "unnormalised"
    # raw q, k: each group's rows are normalised into its share of the workspace
    Qr, Kr = Q * 1.5, K * 0.75
    wn = ops.tt_prefill_normed_workspace_bytes(B, H, N, dk, 64, n)
    wg = ops.tt_prefill_normed_workspace_bytes(1, group, N, dk, 64, n)
    assert wg < wn
    small_n = torch.empty(wg, dtype=torch.uint8, device="cuda")
    O4_ref, S4_ref = ops.tt_prefill_normed(Qr, Kr, V, n, 0.9, states_in=S_ref)
    O4, S4 = ops.tt_prefill_normed(Qr, Kr, V, n, 0.9, states_in=S_ref, workspace=small_n)
    torch.cuda.synchronize()
    assert torch.equal(O4, O4_ref) and torch.equal(S4, S4_ref), "normalised"


def test_head_groups_refuse_less_than_one_head():
    import torch
    B, H, N, dk, n = 1, 3, 1100, 64, 3
    q, k, v = wl.draw_qkv(5200, B, H, N, dk, 64, "bf16")
    Q, K, V = to_device(q), to_device(k), to_device(v)
    need = ops.tt_prefill_workspace_bytes_dtype(B, H, N, dk, 64, n, 64, "bf16")
    tiny = torch.empty(need // (B * H) - 256, dtype=torch.uint8, device="cuda")
    O = torch.zeros((B, H, N, 64), device="cuda")
    with pytest.raises(ops.TTError) as e:
        ops.tt_prefill(Q, K, V, n, O=O, workspace=tiny)
    assert e.value.code == ops.TT_ERR_WORKSPACE and "per head" in str(e.value)
    # the normalised prefill: less than one head's share of its workspace
    w1 = ops.tt_prefill_normed_workspace_bytes(1, 1, N, dk, 64, n)
    half = torch.empty(w1 // 2, dtype=torch.uint8, device="cuda")
    with pytest.raises(ops.TTError) as e:
        ops.tt_prefill_normed(Q, K, V, n, 1.0, O=O, workspace=half)
    assert e.value.code == ops.TT_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert not O.abs().max().item()  # nothing ran


@pytest.mark.parametrize("B,H,N,dk,n,dtype,group", [(1, 16, 65536, 64, 3, "bf16", 2), (1, 16, 16384, 16, 5, "f32", 4)])
def test_head_groups_at_full_size(B, H, N, dk, n, dtype, group):
    """The wide-key (dk 64, 65,536 tokens) and order-5 workloads at their
    full sizes with a workspace of at most 100 MB (2 and 4 heads per group):
    bit-identical to the whole workspace."""
    import torch
    print(f"\n[groups full size] B{B} H{H} N{N} dk{dk} n{n} {dtype}, {group} heads per group", flush=True)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda")
    g.manual_seed(5300 + dk)
    Q = torch.nn.functional.normalize(torch.randn((B, H, N, dk), generator=g, device="cuda"), dim=-1).to(dt)
    K = torch.nn.functional.normalize(torch.randn((B, H, N, dk), generator=g, device="cuda"), dim=-1).to(dt)
    V = torch.randn((B, H, N, 64), generator=g, device="cuda").to(dt)
    per_head = ops.tt_prefill_workspace_bytes_dtype(1, 1, N, dk, 64, n, 64, dtype)
    assert per_head * group <= 100_000_000
    O_ref, S_ref = ops.tt_prefill(Q, K, V, n)
    ws = torch.empty(per_head * group, dtype=torch.uint8, device="cuda")
    O, S = ops.tt_prefill(Q, K, V, n, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(O, O_ref) and torch.equal(S, S_ref)


def test_binding_caps_the_workspace_it_allocates():
    """max_workspace_bytes: the binding allocates at most that much; a
    streamed plan then runs in head groups (same results), a sweep plan
    refuses the capped workspace."""
    import torch
    B, H, N, dk, n = 1, 4, 1500, 64, 3
    print(f"\n[groups via the binding] B{B} H{H} N{N} dk{dk} n{n} bf16", flush=True)
    q, k, v = wl.draw_qkv(5400, B, H, N, dk, 64, "bf16")
    Q, K, V = to_device(q), to_device(k), to_device(v)
    per_head = ops.tt_prefill_workspace_bytes_dtype(1, 1, N, dk, 64, n, 64, "bf16")
    O_ref, S_ref = ops.tt_prefill(Q, K, V, n)
    O, S = ops.tt_prefill(Q, K, V, n, max_workspace_bytes=per_head * 3)
    O2_ref, S2_ref = ops.tt_prefill_from(Q, K, V, S_ref, n)
    O2, S2 = ops.tt_prefill_from(Q, K, V, S_ref, n, max_workspace_bytes=per_head)
    w1 = ops.tt_prefill_normed_workspace_bytes(1, 1, N, dk, 64, n)
    O3_ref, S3_ref = ops.tt_prefill_normed(Q, K, V, n, 1.2)
    O3, S3 = ops.tt_prefill_normed(Q, K, V, n, 1.2, max_workspace_bytes=w1 * 2)
    torch.cuda.synchronize()
    assert torch.equal(O, O_ref) and torch.equal(S, S_ref)
    assert torch.equal(O2, O2_ref) and torch.equal(S2, S2_ref)
    assert torch.equal(O3, O3_ref) and torch.equal(S3, S3_ref)
    with pytest.raises(ops.TTError) as e:  # the chunk-32 sweep: whole workspace only
        ops.tt_prefill(Q, K, V, n, 32, max_workspace_bytes=per_head)
    assert e.value.code == ops.TT_ERR_WORKSPACE
    with pytest.raises(ValueError):
        ops.tt_prefill(Q, K, V, n, max_workspace_bytes=0)
