"""Non-finite inputs and the zero normaliser on the GPU, against the
row-sliced fp64 oracle (row i sums over keys j <= i only).

The definition ("Expanding Attention: A Taylor-Series Route to Linear-Time
Transformers with a Fixed Number of Recurrent States", abstract: softmax
with exp replaced by its n-term Taylor series; the normaliser is the extra
"+1" state column of the comment thread on item 46888355) makes a NaN or
Inf in token j reach the outputs of tokens i >= j only.  The library keeps
that for every output of an earlier chunk of 64 tokens and for the states;
inside the chunk that holds j, a non-finite value v_j can also reach the
outputs of the earlier queries of that chunk in the columns where v_j is not
finite (the masked zero weights of the intra-chunk product multiply v_j).

n = 2 has K_2(-1) = 0: with q = e_0 and every key -e_0 every weight is zero,
the normaliser is exactly zero, and the output is 0/0 = NaN.
"""
import numpy as np
import pytest

import oracle.taylor_oracle as orc
from gpu_util import assert_out
from taylor_recurrent_states_amd import ops

pytestmark = pytest.mark.gpu

CH = 64


def _dev(x64, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda(), t.to(torch.float64).numpy()


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _tol(dtype):
    return ("rel", 1e-5) if dtype == "f32" else ("abs", 5e-3)


@pytest.mark.parametrize("dk,n", [(16, 3), (64, 3), (16, 5)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_value_reaches_later_tokens_only(dk, n, dtype):
    """v_j[5] = NaN at j = 100 of 1000 tokens (16 spans of 64 tokens): every
    output before j's chunk and every column other than 5 matches the
    oracle; column 5 is NaN from token j on; value-plane column 5 of the
    states is NaN, everything else in the states is finite."""
    import torch
    B, H, N, dv, j, col = 1, 1, 1000, 64, 100, 5
    print(f"\n[nonfinite] nan value dk{dk} n{n} {dtype}", flush=True)
    rng = np.random.default_rng(7000 + dk + n)
    q64 = _unit(rng.standard_normal((B, H, N, dk)))
    k64 = _unit(rng.standard_normal((B, H, N, dk)))
    v64 = rng.standard_normal((B, H, N, dv))
    v64[0, 0, j, col] = np.nan
    q, qx = _dev(q64, dtype)
    k, kx = _dev(k64, dtype)
    v, vx = _dev(v64, dtype)
    O, S = ops.tt_prefill(q, k, v, n)
    torch.cuda.synchronize()
    O = O.cpu().numpy()[0, 0]
    ref = orc.quadratic_attention(qx, kx, vx, n)[0, 0]
    assert np.all(np.isnan(ref[j:, col])) and np.all(np.isfinite(ref[:j, col]))
    other = [c for c in range(dv) if c != col]
    assert_out(O[:, other], ref[:, other], _tol(dtype), "columns without the NaN")
    c0 = j // CH * CH  # first token of j's chunk
    assert_out(O[:c0, col], ref[:c0, col], _tol(dtype), "column 5 before the chunk of j")
    assert np.all(np.isnan(O[j:, col]))
    W = ops.tt_state_rows(dk, n)
    st = orc.planes_to_states(S.cpu().numpy(), 1, 1, W, dv)[0, 0]
    assert np.all(np.isnan(st[:, col]))  # every mu_t(k_j) is nonzero for a random unit key
    assert np.all(np.isfinite(st[:, other])) and np.all(np.isfinite(st[:, dv]))


@pytest.mark.parametrize("dk,n", [(16, 3), (64, 3)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_inf_key_reaches_later_tokens_only(dk, n, dtype):
    """k_j[0] = +Inf at j = 150: outputs before j match the oracle (the
    masked weights of the intra-chunk block are selected to zero, not
    multiplied); from j on, the oracle and the library are not finite."""
    import torch
    B, H, N, dv, j = 1, 1, 700, 64, 150
    print(f"\n[nonfinite] inf key dk{dk} n{n} {dtype}", flush=True)
    rng = np.random.default_rng(7100 + dk + n)
    q64 = _unit(rng.standard_normal((B, H, N, dk)))
    k64 = _unit(rng.standard_normal((B, H, N, dk)))
    k64[0, 0, j, 0] = np.inf
    v64 = rng.standard_normal((B, H, N, dv))
    q, qx = _dev(q64, dtype)
    k, kx = _dev(k64, dtype)
    v, vx = _dev(v64, dtype)
    O, _ = ops.tt_prefill(q, k, v, n)
    torch.cuda.synchronize()
    O = O.cpu().numpy()[0, 0]
    with np.errstate(all="ignore"):
        ref = orc.quadratic_attention(qx, kx, vx, n)[0, 0]
    assert np.all(~np.isfinite(ref[j:]).all(axis=1))
    assert_out(O[:j], ref[:j], _tol(dtype), "before the Inf key")
    assert np.all(~np.isfinite(O[j:]).all(axis=1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_propagates_nan(dtype):
    """A NaN value in one decode step makes that head's value column NaN in
    the output and the states; other heads are untouched."""
    import torch
    B, H, dk, dv, n = 1, 4, 16, 64, 3
    rng = np.random.default_rng(7200)
    S0 = orc.states_definition(_unit(rng.standard_normal((B, H, 50, dk))), rng.standard_normal((B, H, 50, dv)), n)
    S = torch.from_numpy(orc.states_to_planes(S0).astype(np.float32)).cuda()
    q, qx = _dev(_unit(rng.standard_normal((B, H, dk))), dtype)
    k, kx = _dev(_unit(rng.standard_normal((B, H, dk))), dtype)
    v64 = rng.standard_normal((B, H, dv))
    v64[0, 2, 7] = np.nan
    v, vx = _dev(v64, dtype)
    o = ops.tt_decode_step(q, k, v, S, n)
    torch.cuda.synchronize()
    o_ref, _ = orc.decode_step(qx, kx, vx, S0.astype(np.float32).astype(np.float64), n)
    o = o.cpu().numpy()
    assert np.isnan(o[0, 2, 7]) and np.isnan(o_ref[0, 2, 7])
    fin = np.isfinite(o_ref)
    assert fin.sum() == o.size - 1
    assert_out(o[fin], o_ref[fin], ("rel", 1e-5) if dtype == "f32" else ("abs", 5e-3), "finite outputs")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_normaliser_gives_nan(dtype):
    """n = 2, q = e_0 and every key -e_0: K_2(q.k) = 1 - 1 = 0 for every
    pair, so every output is 0/0 (oracle: NaN).  fp32 over several chunks
    and spans and a decode step after it; bf16 within one chunk (its
    readout of the state rounds S to bf16, so across chunks the normaliser
    is a rounding residue rather than an exact zero)."""
    import torch
    B, H, dk, dv, n = 1, 2, 16, 64, 2
    N = 300 if dtype == "f32" else CH
    rng = np.random.default_rng(7300)
    e = np.eye(dk)
    q, qx = _dev(np.broadcast_to(e[0], (B, H, N, dk)), dtype)
    k, kx = _dev(np.broadcast_to(-e[0], (B, H, N, dk)), dtype)
    v, vx = _dev(rng.standard_normal((B, H, N, dv)), dtype)
    O, S = ops.tt_prefill(q, k, v, n)
    with np.errstate(all="ignore"):
        ref = orc.quadratic_attention(qx, kx, vx, n)
    assert np.all(np.isnan(ref))
    torch.cuda.synchronize()
    assert torch.isnan(O).all(), f"{int((~torch.isnan(O)).sum())} outputs are not NaN"
    if dtype == "f32":
        o = ops.tt_decode_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous(), S, n)
        torch.cuda.synchronize()
        assert torch.isnan(o).all()
