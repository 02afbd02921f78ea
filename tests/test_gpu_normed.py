"""GPU parity of the normalised path (L2 normalisation of q and k with a
temperature on the queries) against the fp64 oracle.

"Expanding Attention" (abstract) makes unit q and k the prerequisite of the
method; the oracle's ``normalized_inputs`` normalises raw rows in fp64 (the
plain definition) and rounds them to the input dtype the way the inputs are
rounded.  The library evaluates the quotient in fp64 as well, so:

* tt_normalize_rows equals the oracle's rounded unit rows bit for bit,
  except where the oracle's fp64 value lies within 2^-45 (relative) of a
  rounding boundary; there either neighbour is a correct rounding of the
  exact value (both fp64 evaluations are within about 2^-49 of it) and the
  test accepts either;
* the temperature crosses the C boundary as a float, so the oracle is given
  that fp32 value (``_t32``);
* tt_prefill_normed / tt_decode_step_normed on raw inputs meet the parity
  bar of the plain path (fp32 1e-5 relative, bf16 5e-3 absolute) against
  the oracle's attention on its normalised rows.
"""
import numpy as np
import pytest

import oracle.taylor_oracle as orc
from gpu_util import assert_out, assert_states, to_device
from taylor_recurrent_states_amd import ops
from taylor_recurrent_states_amd import workloads as wl

pytestmark = pytest.mark.gpu

SHAPES = [(16, 1), (16, 2), (16, 3), (16, 4), (16, 5), (32, 1), (32, 2), (32, 3), (32, 4), (64, 1), (64, 2), (64, 3),
          (64, 4)]


def _tol(dtype):
    return ("rel", 1e-5) if dtype == "f32" else ("abs", 5e-3)


def _t32(tau):
    """The temperature the library receives: the C ``float`` nearest tau."""
    return float(np.float32(tau))


def _raw(seed, B, H, N, dk, dv, dtype):
    """Raw Gaussian q, k (norms spread over two decades) and v, rounded to dtype."""
    q, k, v = wl.draw_qkv(seed, B, H, N, dk, dv, "f32", normalise=False)
    g = np.random.Generator(np.random.PCG64([seed, 5]))
    sq = 10.0 ** g.uniform(-1, 1, (B, H, N, 1))
    sk = 10.0 ** g.uniform(-1, 1, (B, H, N, 1))
    return wl.round_to(q.exact * sq, dtype), wl.round_to(k.exact * sk, dtype), wl.round_to(v.exact, dtype)


@pytest.mark.parametrize("d", [8, 16, 32, 64])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tau", [1.0, 0.7])
def test_normalize_rows(d, dtype, tau):
    import torch
    rows = 1000
    x, _, _ = _raw(500 + d, 1, 1, rows, d, 4, dtype)
    xd = to_device(x)[0, 0]
    got = ops.tt_normalize_rows(xd, tau)
    g = got.float().cpu().numpy().astype(np.float64)
    exact = orc.normalize_rows(x.exact[0, 0], _t32(tau))
    ref = orc.round_to_dtype(exact, dtype)
    # where the fp64 value is that close to a rounding boundary, both
    # neighbours are correct roundings of the exact quotient
    lo = orc.round_to_dtype(exact * (1 - 2.0 ** -45), dtype)
    hi = orc.round_to_dtype(exact * (1 + 2.0 ** -45), dtype)
    sure = lo == hi
    assert np.array_equal(g[sure], ref[sure]), f"{np.sum(g[sure] != ref[sure])} of {int(sure.sum())} values differ"
    assert np.all((g == lo) | (g == hi))
    assert np.sum(~sure) <= 2, f"{np.sum(~sure)} coordinates lie on a rounding boundary"
    # in place gives the same bits
    y = xd.clone()
    ops.tt_normalize_rows(y, tau, out=y)
    assert torch.equal(y, got)
    # a zero row has no direction
    z = torch.zeros((3, d), dtype=xd.dtype, device=xd.device)
    assert torch.isnan(ops.tt_normalize_rows(z, tau).float()).all()
    torch.cuda.synchronize()


@pytest.mark.parametrize("dk,n", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_normed_small(dk, n, dtype):
    import torch
    B, H, N = 1, 2, 200  # three full chunks and a ragged tail
    q, k, v = _raw(4100 + dk * 10 + n, B, H, N, dk, 64, dtype)
    taus = [1.0, 0.5] + ([1.5] if n % 2 == 1 else [])  # K_n > 0 on all of R for odd n
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    for tau in taus:
        O, S = ops.tt_prefill_normed(Qd, Kd, Vd, n, tau)
        torch.cuda.synchronize()
        qh, kh = orc.normalized_inputs(q.exact, k.exact, _t32(tau), dtype)
        assert_out(O.cpu().numpy(), orc.quadratic_attention(qh, kh, v.exact, n), _tol(dtype), f"dk{dk} n{n} tau{tau}")
        assert_states(S.cpu().numpy(), orc.states_definition(kh, v.exact, n), dk, n, _tol(dtype),
                      f"dk{dk} n{n} tau{tau}")
    # raw inputs are read-only
    assert torch.equal(Qd, to_device(q)) and torch.equal(Kd, to_device(k))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_normed_equals_prefill_on_normalised_rows(dtype):
    """The normalised prefill is tt_prefill on tt_normalize_rows' output, bit for bit."""
    import torch
    B, H, N, dk, n, tau = 2, 3, 333, 16, 3, 0.8
    q, k, v = _raw(4200, B, H, N, dk, 64, dtype)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    O1, S1 = ops.tt_prefill_normed(Qd, Kd, Vd, n, tau)
    Qn = ops.tt_normalize_rows(Qd.reshape(-1, dk), tau).reshape(Qd.shape)
    Kn = ops.tt_normalize_rows(Kd.reshape(-1, dk), 1.0).reshape(Kd.shape)
    O2, S2 = ops.tt_prefill(Qn, Kn, Vd, n)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_normed_from_states_then_decode(dtype):
    """Carried-in states, then decode steps on raw inputs: every output and
    the final states against the oracle on the normalised rows."""
    import torch
    B, H, P, N, dk, n, tau = 2, 2, 100, 190, 16, 3, 0.9
    qp, kp, vp = _raw(4300, B, H, P, dk, 64, dtype)
    _, kph = orc.normalized_inputs(qp.exact, kp.exact, _t32(tau), dtype)
    S0 = orc.states_definition(kph, vp.exact, n).astype(np.float32).astype(np.float64)
    S0d = torch.from_numpy(orc.states_to_planes(S0).astype(np.float32)).cuda()
    q, k, v = _raw(4301, B, H, N, dk, 64, dtype)
    O, S = ops.tt_prefill_normed(to_device(q), to_device(k), to_device(v), n, tau, states_in=S0d)
    torch.cuda.synchronize()
    qh, kh = orc.normalized_inputs(q.exact, k.exact, _t32(tau), dtype)
    o_ref, S_ref = orc.prefill_from_states(qh, kh, v.exact, S0, n)
    assert_out(O.cpu().numpy(), o_ref, _tol(dtype), "prefill_normed from states")
    assert_states(S.cpu().numpy(), S_ref, dk, n, _tol(dtype), "prefill_normed from states")
    # continue with decode steps on raw tokens
    S_run = S.cpu().numpy().astype(np.float64)
    S_log = orc.planes_to_states(S_run, B, H, orc.state_rows(dk, n), 64)
    for t in range(4):
        qt, kt, vt = _raw(4400 + t, B, H, 1, dk, 64, dtype)
        o = ops.tt_decode_step_normed(to_device(qt)[:, :, 0].contiguous(), to_device(kt)[:, :, 0].contiguous(),
                                      to_device(vt)[:, :, 0].contiguous(), S, n, tau)
        torch.cuda.synchronize()
        qth, kth = orc.normalized_inputs(qt.exact[:, :, 0], kt.exact[:, :, 0], _t32(tau), dtype)
        o_ref, S_log = orc.decode_step(qth, kth, vt.exact[:, :, 0], S_log, n)
        assert_out(o.cpu().numpy(), o_ref, _tol(dtype), f"decode_normed step {t}")
    assert_states(S.cpu().numpy(), S_log, dk, n, _tol(dtype), "after decode_normed")


@pytest.mark.parametrize("dk,n", [(32, 3), (32, 4), (64, 4)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_normed_continues_prefill_normed(dk, n, dtype):
    """Prefill of N tokens then one decode step equals the prefill of N+1
    tokens on the last output and the states (both normalise with the same
    device function).  dk 64 n 4 (47,905 rows) runs the decode over row
    chunks."""
    import torch
    B, H, N, tau = 1, 4, 129, 1.0
    q, k, v = _raw(4500 + dk * 10 + n, B, H, N + 1, dk, 64, dtype)
    Qd, Kd, Vd = to_device(q), to_device(k), to_device(v)
    O_all, S_all = ops.tt_prefill_normed(Qd, Kd, Vd, n, tau)
    _, S = ops.tt_prefill_normed(Qd[:, :, :N].contiguous(), Kd[:, :, :N].contiguous(), Vd[:, :, :N].contiguous(),
                                 n, tau)
    o = ops.tt_decode_step_normed(Qd[:, :, N].contiguous(), Kd[:, :, N].contiguous(), Vd[:, :, N].contiguous(),
                                  S, n, tau)
    torch.cuda.synchronize()
    # the bf16 prefill reads out through bf16 MFMA operands, the decode in fp32:
    # both are held to the parity bar of their dtype
    assert_out(o.cpu().numpy(), O_all[:, :, N].cpu().numpy(), _tol(dtype), "decode vs prefill, last token")
    sa, sb = S.cpu().numpy().astype(np.float64), S_all.cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(sa - sb)))
    assert err <= 1e-5 * float(np.max(np.abs(sb))), err


def test_prefill_normed_full_size():
    """The prefill workload's shape (B4 H8 N8192 dk16 bf16, n = 3) on raw
    inputs: every state element and sampled output rows of all heads."""
    import torch
    w = wl.WORKLOADS["prefill"]
    tau = 1.0
    print("\n[prefill_normed] drawing inputs", flush=True)
    q, k, v = _raw(w.seed, w.B, w.H, w.N, w.dk, w.dv, w.dtype)
    O, S = ops.tt_prefill_normed(to_device(q), to_device(k), to_device(v), w.n, tau, chunk=w.chunk)
    torch.cuda.synchronize()
    O, S = O.cpu().numpy(), S.cpu().numpy()
    print("[prefill_normed] GPU done", flush=True)
    qh, kh = orc.normalized_inputs(q.exact, k.exact, _t32(tau), w.dtype)
    BH = w.B * w.H
    assert_states(S, orc.states_definition(kh, v.exact, w.n), w.dk, w.n, w.tol, "prefill_normed")
    rng = np.random.Generator(np.random.PCG64([w.seed, 98]))
    Qx, Kx, Vx = qh.reshape(BH, w.N, w.dk), kh.reshape(BH, w.N, w.dk), v.exact.reshape(BH, w.N, w.dv)
    Og = O.reshape(BH, w.N, w.dv)
    for h in range(BH):
        rows = sorted({0, 1, 63, 64, 65, w.N - 1} | set(int(r) for r in rng.integers(0, w.N, 10)))
        ref = orc.quadratic_rows(Qx[h, rows], Kx[h], Vx[h], rows, w.n)
        assert_out(Og[h, rows], ref, w.tol, f"prefill_normed head {h}")
