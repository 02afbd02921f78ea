"""GPU parity of tt_prefill (and its composition with decode and merge)
against the fp64 oracle.

Bar: fp32 inputs 1e-5 relative (max|x - ref| / max|ref| per tensor, per
(m-block, plane) for states); bf16 inputs 5e-3 absolute.  Small cases are
compared element by element against the quadratic form; the full-size
workloads compare every state element and sampled output rows (the oracle
evaluates those rows one by one from the definition).
"""
import dataclasses

import numpy as np
import pytest

import oracle.taylor_oracle as orc
from gpu_util import assert_out, assert_states, oracle_rows, oracle_states, to_device
from taylor_recurrent_states_amd import ops
from taylor_recurrent_states_amd import workloads as wl

pytestmark = pytest.mark.gpu

SHAPES = [(16, 1), (16, 2), (16, 3), (16, 4), (16, 5), (32, 1), (32, 2), (32, 3), (64, 1), (64, 2), (64, 3)]


def _tol(dtype):
    return ("rel", 1e-5) if dtype == "f32" else ("abs", 5e-3)


def _prefill(q, k, v, n):
    import torch
    O, S = ops.tt_prefill(to_device(q), to_device(k), to_device(v), n, 64)
    torch.cuda.synchronize()
    return O.cpu().numpy(), S.cpu().numpy()


@pytest.mark.parametrize("dk,n", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_small(dk, n, dtype):
    B, H, N = 1, 2, 200  # three full chunks and a ragged tail
    q, k, v = wl.draw_qkv(1000 + dk * 10 + n, B, H, N, dk, 64, dtype)
    O, S = _prefill(q, k, v, n)
    assert_out(O, orc.quadratic_attention(q.exact, k.exact, v.exact, n), _tol(dtype), f"dk{dk} n{n}")
    assert_states(S, orc.states_definition(k.exact, v.exact, n), dk, n, _tol(dtype), f"dk{dk} n{n}")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_prefill_small_dk8(n):
    """dk = 8 (fp32 inputs), up to six Taylor terms: C(13, 5) = 1287 feature
    rows at n = 6."""
    B, H, N, dk = 1, 2, 200, 8
    q, k, v = wl.draw_qkv(1500 + n, B, H, N, dk, 64, "f32")
    O, S = _prefill(q, k, v, n)
    assert_out(O, orc.quadratic_attention(q.exact, k.exact, v.exact, n), _tol("f32"), f"dk8 n{n}")
    assert_states(S, orc.states_definition(k.exact, v.exact, n), dk, n, _tol("f32"), f"dk8 n{n}")


def test_prefill_dk8_bf16_is_unsupported():
    q, k, v = wl.draw_qkv(1600, 1, 1, 64, 8, 64, "bf16")
    with pytest.raises(ops.TTError) as e:
        ops.tt_prefill(to_device(q), to_device(k), to_device(v), 3)
    assert e.value.code == ops.TT_ERR_UNSUPPORTED


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 128, 129, 300, 1000])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_lengths(N, dtype):
    B, H, dk, n = 2, 3, 16, 3
    q, k, v = wl.draw_qkv(2000 + N, B, H, N, dk, 64, dtype)
    O, S = _prefill(q, k, v, n)
    assert_out(O, orc.quadratic_attention(q.exact, k.exact, v.exact, n), _tol(dtype), f"N{N}")
    assert_states(S, orc.states_definition(k.exact, v.exact, n), dk, n, _tol(dtype), f"N{N}")


def test_tiny_workload():
    """Single sequence, one head, N=256, dk=16, dv=64, n=3, seed 0, fp32."""
    w = wl.WORKLOADS["tiny"]
    q, k, v = wl.draw_qkv(w.seed, w.B, w.H, w.N, w.dk, w.dv, w.dtype)
    O, S = _prefill(q, k, v, w.n)
    assert_out(O, orc.quadratic_attention(q.exact, k.exact, v.exact, w.n), w.tol)
    assert_states(S, orc.states_definition(k.exact, v.exact, w.n), w.dk, w.n, w.tol)


def _sample_rows(N, rng, extra=24):
    base = {0, 1, 2, 31, 32, 63, 64, 65, 127, 128, N // 2, N // 2 + 1, N - 65, N - 64, N - 2, N - 1}
    # both sides of every multiple of 512 tokens: the span boundaries of the
    # full-size plans (spans of 512 or 1024 tokens)
    base |= {r for m in range(512, N, 512) for r in (m - 1, m)}
    base |= set(int(x) for x in rng.integers(0, N, extra))
    return sorted(r for r in base if 0 <= r < N)


def _full_workload(name, heads_checked=None, state_heads=None, w=None, vmap=None):
    """Run the named workload (or ``w``) at full size; compare sampled output
    rows of ``heads_checked`` (default: all heads) and every state element of
    ``state_heads`` (default: the same heads) against the oracle.  ``vmap``
    transforms the drawn values (fp64) before they are rounded again."""
    w = wl.WORKLOADS[name] if w is None else w
    print(f"\n[{name}] drawing inputs", flush=True)
    q, k, v = wl.draw_qkv(w.seed, w.B, w.H, w.N, w.dk, w.dv, w.dtype)
    if vmap is not None:
        v = wl.round_to(vmap(v.exact), w.dtype)
    O, S = _prefill(q, k, v, w.n)
    print(f"[{name}] GPU prefill done", flush=True)
    rng = np.random.Generator(np.random.PCG64([w.seed, 99]))
    BH = w.B * w.H
    Qx = q.exact.reshape(BH, w.N, w.dk)
    Kx = k.exact.reshape(BH, w.N, w.dk)
    Vx = v.exact.reshape(BH, w.N, w.dv)
    Og = O.reshape(BH, w.N, w.dv)
    heads = list(range(BH)) if heads_checked is None else list(heads_checked)
    rows_of = {h: _sample_rows(w.N, rng) for h in heads}
    refs = oracle_rows(Qx, Kx, Vx, rows_of, w.n, heads)
    worst = 0.0
    for h, ref in zip(heads, refs):
        worst = max(worst, assert_out(Og[h, rows_of[h]], ref, w.tol, f"{name} head {h}"))
    print(f"[{name}] sampled rows of {len(heads)} heads ok (worst {worst:.2e})", flush=True)
    W = orc.state_rows(w.dk, w.n)
    heads = heads if state_heads is None else list(state_heads)
    S_got = orc.planes_to_states(S, 1, BH, W, w.dv)[0][heads]
    S_ref = np.stack(oracle_states(Kx, Vx, w.n, heads))
    errs = assert_states(orc.states_to_planes(S_got[None]), S_ref[None], w.dk, w.n, w.tol, name)
    print(f"[{name}] states of {len(heads)} heads ok", flush=True)
    return q, k, v, S, S_ref, heads, errs


def test_prefill_workload_full_size():
    """B=4, H=8, N=8192, dk=16, n=3, bf16: every state element, sampled rows of every head."""
    _full_workload("prefill")


@pytest.mark.parametrize("shift,scale", [(3.0, 1.0), (0.0, 4.0)])
def test_prefill_workload_full_size_offset_values(shift, scale):
    """The prefill workload with values shift + scale * N(0, 1): outputs
    near 3, or four times the spread, where the bf16 readout of the state
    is weakest.  Every state element, sampled rows of every head."""
    w = dataclasses.replace(wl.WORKLOADS["prefill"], name=f"prefill v~{shift}+{scale}N(0,1)", seed=21)
    _full_workload(w.name, w=w, vmap=lambda x: shift + scale * x)


@pytest.mark.parametrize("B,H,N", [(4, 8, 8155), (2, 8, 8129)])
def test_prefill_workload_ragged_length(B, H, N):
    """The prefill workload's shape with a length that ends inside a chunk.
    With B*H = 32 the plan has 8 spans of 1024 tokens and the last one ends
    27 tokens into its final chunk; with B*H = 16 it has 16 spans of 512 and
    the last ends 1 token into its final chunk.  Sampled rows of every head
    (span boundaries and the ragged tail included) and every state element
    of every head."""
    w = dataclasses.replace(wl.WORKLOADS["prefill"], name=f"prefill B{B} H{H} N{N}", B=B, H=H, N=N, seed=11)
    _full_workload(w.name, w=w)


@pytest.mark.timeout(600)
def test_order5_workload_full_size():
    """B=1, H=16, N=16384, dk=16, n=5, fp32: sampled rows and every state
    element of every head."""
    _full_workload("order5")


@pytest.mark.timeout(600)
def test_wide_workload_full_size_and_split_merge():
    """B=1, H=16, N=65536, dk=64, n=3, bf16: sampled rows and every state
    element of every head; then the states of 8 random chunk splits merged
    with tt_state_merge equal the single pass (GPU vs GPU) and the oracle, on
    every head."""
    import torch
    w = wl.WORKLOADS["wide"]
    q, k, v, S_single, S_ref, heads, _ = _full_workload("wide")
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    cuts = [0] + wl.draw_split_points(w.N, w.extra["splits"] - 1) + [w.N]
    merged = None
    for a, b in zip(cuts[:-1], cuts[1:]):
        _, S = ops.tt_prefill(Qd[:, :, a:b].contiguous(), Kd[:, :, a:b].contiguous(), Vd[:, :, a:b].contiguous(),
                              w.n, 64)
        merged = S if merged is None else ops.tt_state_merge(merged, S)
    torch.cuda.synchronize()
    m = merged.cpu().numpy()
    print(f"[wide] merged {len(cuts) - 1} splits at {cuts[1:-1]}", flush=True)
    assert np.max(np.abs(m - S_single)) <= 5e-3
    W = orc.state_rows(w.dk, w.n)
    m_heads = orc.planes_to_states(m, 1, w.B * w.H, W, w.dv)[0][list(heads)]
    assert_states(orc.states_to_planes(m_heads[None]), S_ref[None], w.dk, w.n, w.tol, "merged splits")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_then_decode_equals_longer_prefill(dtype):
    """Prefill of N tokens, then decode steps, reproduce the prefill of the
    whole sequence (outputs at the decoded positions and final states)."""
    import torch
    B, H, N, extra, dk, n = 2, 2, 150, 6, 16, 3
    q, k, v = wl.draw_qkv(31, B, H, N + extra, dk, 64, dtype)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    _, S = ops.tt_prefill(Qd[:, :, :N].contiguous(), Kd[:, :, :N].contiguous(), Vd[:, :, :N].contiguous(), n)
    outs = []
    for t in range(N, N + extra):
        outs.append(ops.tt_decode_step(Qd[:, :, t].contiguous(), Kd[:, :, t].contiguous(), Vd[:, :, t].contiguous(),
                                       S, n).cpu().numpy())
    torch.cuda.synchronize()
    ref = orc.quadratic_attention(q.exact, k.exact, v.exact, n)[:, :, N:]
    assert_out(np.stack(outs, axis=2), ref, _tol(dtype))
    assert_states(S.cpu().numpy(), orc.states_definition(k.exact, v.exact, n), dk, n, _tol(dtype))


@pytest.mark.parametrize("dk,n", [(16, 3), (32, 2), (16, 4)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_equals_decode_steps_from_zero(dk, n, dtype):
    """The chunked prefill and N single-token decode steps from zero states
    are two paths to the same outputs and states (cross-path check); both
    are held to the parity bar against each other."""
    import torch
    B, H, N = 1, 2, 130
    q, k, v = wl.draw_qkv(41 + dk + n, B, H, N, dk, 64, dtype)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    O, S = ops.tt_prefill(Qd, Kd, Vd, n)
    Sd = torch.zeros_like(S)
    outs = [ops.tt_decode_step(Qd[:, :, t].contiguous(), Kd[:, :, t].contiguous(), Vd[:, :, t].contiguous(), Sd,
                               n).cpu().numpy() for t in range(N)]
    torch.cuda.synchronize()
    O_dec = np.stack(outs, axis=2)
    assert_out(O.cpu().numpy(), O_dec, _tol(dtype), f"prefill vs decode dk{dk} n{n}")
    W = orc.state_rows(dk, n)
    S_dec = orc.planes_to_states(Sd.cpu().numpy().astype(np.float64), B, H, W, 64)
    assert_states(S.cpu().numpy(), S_dec, dk, n, _tol(dtype), f"prefill vs decode dk{dk} n{n}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_independent_of_span_split(dtype):
    """Two heads prefilled alone (64 spans of one chunk each) and the same
    two heads inside a 32-head batch (8 spans of 8 chunks): the split of the
    sequence into spans changes only the rounding (the states add), so the
    two results agree to the parity bar, and both match the oracle."""
    import torch
    N, dk, n = 4096, 16, 3
    q, k, v = wl.draw_qkv(43, 1, 2, N, dk, 64, dtype)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    O1, S1 = ops.tt_prefill(Qd, Kd, Vd, n)
    rep = lambda X: X.repeat(1, 16, 1, 1).contiguous()
    O2, S2 = ops.tt_prefill(rep(Qd), rep(Kd), rep(Vd), n)
    torch.cuda.synchronize()
    O1, O2 = O1.cpu().numpy(), O2.cpu().numpy()
    assert_out(O2[:, :2], O1, _tol(dtype), "span split")
    nf = ops.tt_state_floats(dk, 64, n)
    W = orc.state_rows(dk, n)
    S2l = orc.planes_to_states(S2.cpu().numpy().astype(np.float64), 1, 32, W, 64)[:, :2]
    assert_states(S1.cpu().numpy(), S2l, dk, n, _tol(dtype), "span split")
    assert nf == W * 65
    rows = [0, 1, 63, 64, 65, 1000, 2047, 2048, N - 1]
    ref = np.stack([orc.quadratic_rows(q.exact[0, h, rows], k.exact[0, h], v.exact[0, h], rows, n) for h in range(2)])
    assert_out(O1[0][:, rows], ref, _tol(dtype), "alone vs oracle")
    assert_out(O2[0, :2][:, rows], ref, _tol(dtype), "batched vs oracle")


def test_prefill_bitwise_repeatable_and_workspace_reuse():
    import torch
    q, k, v = wl.draw_qkv(5, 2, 4, 777, 16, 64, "bf16")
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    need = ops.tt_prefill_workspace_bytes(2, 4, 777, 16, 64, 3, 64)
    ws = torch.full((need + 4096,), 255, dtype=torch.uint8, device="cuda")  # dirty, oversized
    O1, S1 = ops.tt_prefill(Qd, Kd, Vd, 3, workspace=ws)
    O2, S2 = ops.tt_prefill(Qd, Kd, Vd, 3)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)


def test_prefill_rejects_small_workspace():
    import torch
    q, k, v = wl.draw_qkv(6, 1, 1, 300, 16, 64, "f32")
    need = ops.tt_prefill_workspace_bytes(1, 1, 300, 16, 64, 3, 64)
    if need == 0:
        pytest.skip("no workspace needed")
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ops.TTError) as e:
        ops.tt_prefill(to_device(q), to_device(k), to_device(v), 3, workspace=ws)
    assert e.value.code == ops.TT_ERR_WORKSPACE


@pytest.mark.parametrize("which", ["O"])
def test_prefill_rejects_misaligned_outputs(which):
    """O is written with 16-byte stores: a buffer that is not 16-byte aligned
    is refused before anything is launched."""
    import torch
    q, k, v = wl.draw_qkv(7, 1, 2, 100, 16, 64, "bf16")
    nf = ops.tt_state_floats(16, 64, 3)
    buf_o = torch.empty(1 * 2 * 100 * 64 + 1, dtype=torch.float32, device="cuda")
    buf_s = torch.empty(2 * nf + 1, dtype=torch.float32, device="cuda")
    O = buf_o[1:].view(1, 2, 100, 64) if which == "O" else None
    S = buf_s[1:] if which == "states" else None
    with pytest.raises(ops.TTError) as e:
        ops.tt_prefill(to_device(q), to_device(k), to_device(v), 3, O=O, states=S)
    assert e.value.code == ops.TT_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# Chunk length ("Expanding Attention", abstract: the states add, so the split
# of the sequence into chunks is free; the chunk length moves work between
# the intra-chunk quadratic block and the state readout and update).
# 64 tokens: pipe kernel (bf16, W <= 256) or sweep kernel; 16, 32 and 128:
# sweep kernel compiled per chunk length.  bf16 needs chunks of 32 or more;
# 128-token chunks run the shapes whose tiles fit the LDS of a CU, and the
# others are refused before anything is launched.
# ---------------------------------------------------------------------------

CHUNK_SHAPES = [(8, 6), (16, 1), (16, 3), (16, 5), (32, 2), (64, 3)]


def _refused(dk, n, dtype, chunk):
    """Whether the library refuses the shape, asked without launching: Q is
    misaligned, which the entry point reports (INVALID_ARG) only after the
    plan check (UNSUPPORTED), so the call never reaches a launch."""
    L = ops.lib()
    import ctypes
    misaligned, fake = ctypes.c_void_p(0x1001), ctypes.c_void_p(0x1000)
    rc = L.tt_prefill(misaligned, fake, fake, ops.TT_F32 if dtype == "f32" else ops.TT_BF16, 1, 1, 100, dk, 64, n,
                      chunk, fake, fake, fake, 1 << 40, None)
    assert rc in (ops.TT_ERR_UNSUPPORTED, ops.TT_ERR_INVALID_ARG), rc
    return rc == ops.TT_ERR_UNSUPPORTED


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
@pytest.mark.parametrize("dk,n", CHUNK_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_chunk_lengths(chunk, dk, n, dtype):
    """Every chunk length against the oracle on 300 tokens (ragged for every
    length), B*H = 2, every output and state element."""
    import torch
    B, H, N = 1, 2, 300
    q, k, v = wl.draw_qkv(5000 + 10 * dk + n, B, H, N, dk, 64, dtype)
    if _refused(dk, n, dtype, chunk):
        assert (dtype == "bf16" and (dk < 16 or chunk < 32)) or chunk == 128, "refused unexpectedly"
        with pytest.raises(ops.TTError) as e:
            ops.tt_prefill(to_device(q), to_device(k), to_device(v), n, chunk)
        assert e.value.code == ops.TT_ERR_UNSUPPORTED
        return
    O, S = ops.tt_prefill(to_device(q), to_device(k), to_device(v), n, chunk)
    torch.cuda.synchronize()
    tag = f"chunk{chunk} dk{dk} n{n} {dtype}"
    assert_out(O.cpu().numpy(), orc.quadratic_attention(q.exact, k.exact, v.exact, n), _tol(dtype), tag)
    assert_states(S.cpu().numpy(), orc.states_definition(k.exact, v.exact, n), dk, n, _tol(dtype), tag)


def test_tiny_workload_every_chunk_length():
    """The tiny workload (N = 256, dk 16, n 3, fp32) with chunks of 16, 32,
    64 and 128: each against the quadratic form and the oracle's chunked
    form of the same chunk length, and the four results against each other."""
    import torch
    w = wl.WORKLOADS["tiny"]
    q, k, v = wl.draw_qkv(w.seed, w.B, w.H, w.N, w.dk, w.dv, w.dtype)
    ref = orc.quadratic_attention(q.exact, k.exact, v.exact, w.n)
    outs = {}
    for chunk in (16, 32, 64, 128):
        O, S = ops.tt_prefill(to_device(q), to_device(k), to_device(v), w.n, chunk)
        torch.cuda.synchronize()
        O = O.cpu().numpy()
        o_chunked, _ = orc.chunked_attention(q.exact, k.exact, v.exact, w.n, chunk)
        assert_out(O, ref, w.tol, f"chunk {chunk}")
        assert_out(O, o_chunked, w.tol, f"chunk {chunk} vs chunked oracle")
        assert_states(S.cpu().numpy(), orc.states_definition(k.exact, v.exact, w.n), w.dk, w.n, w.tol, f"chunk {chunk}")
        outs[chunk] = O
    for c in (16, 32, 128):
        assert_out(outs[c], outs[64].astype(np.float64), w.tol, f"chunk {c} vs 64")


def test_prefill_workload_chunk_lengths():
    """The prefill workload (B4 H8 N8192 dk16 n3 bf16) with chunks of 32 and
    128 besides the default 64: sampled rows of every head and every state
    element against the oracle, and all outputs of the three lengths within
    the bar of each other."""
    import torch
    w = wl.WORKLOADS["prefill"]
    print("\n[chunks] drawing inputs", flush=True)
    q, k, v = wl.draw_qkv(w.seed, w.B, w.H, w.N, w.dk, w.dv, w.dtype)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    outs = {}
    for chunk in (32, 64, 128):
        O, S = ops.tt_prefill(Qd, Kd, Vd, w.n, chunk)
        torch.cuda.synchronize()
        outs[chunk] = (O.cpu().numpy(), S.cpu().numpy())
        print(f"[chunks] chunk {chunk} done", flush=True)
    BH = w.B * w.H
    S_ref = orc.states_definition(k.exact, v.exact, w.n)
    rng = np.random.Generator(np.random.PCG64([w.seed, 97]))
    Qx, Kx, Vx = (a.exact.reshape(BH, w.N, -1) for a in (q, k, v))
    for chunk, (O, S) in outs.items():
        assert_states(S, S_ref, w.dk, w.n, w.tol, f"chunk {chunk}")
        Og = O.reshape(BH, w.N, w.dv)
        for h in range(BH):
            rows = _sample_rows(w.N, rng, extra=8)
            ref = orc.quadratic_rows(Qx[h, rows], Kx[h], Vx[h], rows, w.n)
            assert_out(Og[h, rows], ref, w.tol, f"chunk {chunk} head {h}")
        print(f"[chunks] chunk {chunk} against the oracle ok", flush=True)
    for chunk in (32, 128):
        assert_out(outs[chunk][0], outs[64][0].astype(np.float64), w.tol, f"chunk {chunk} vs 64")
