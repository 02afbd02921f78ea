"""Host-side checks of the Python binding: caller-supplied buffers of the
wrong dtype, size or shape are refused with ValueError before any entry
point that launches work is called (the C entry points take raw pointers
and no buffer sizes, so a short output would otherwise be written out of
bounds).  Runs on the CPU: the refusals come before the device checks."""
import pytest
import torch

from taylor_recurrent_states_amd import ops

SIZE_QUERIES = {"tt_state_rows", "tt_state_floats", "tt_prefill_workspace_bytes", "tt_prefill_workspace_bytes_dtype",
                "tt_prefill_normed_workspace_bytes", "tt_softmax_decode_workspace_bytes", "tt_last_error"}


class _Guard:
    """Stands in for the loaded library: size queries go through, any
    entry point that would launch work is recorded."""

    def __init__(self, real):
        self.real = real
        self.launched = []

    def __getattr__(self, name):
        if name in SIZE_QUERIES:
            return getattr(self.real, name)
        self.launched.append(name)
        raise AssertionError(f"{name} called")


@pytest.fixture
def guard(monkeypatch):
    g = _Guard(ops.lib())
    monkeypatch.setattr(ops, "lib", lambda: g)
    yield g
    assert not g.launched, g.launched


def _qkv(B=1, H=2, N=10, dk=16, dv=64, dtype=torch.bfloat16):
    return (torch.zeros(B, H, N, dk, dtype=dtype), torch.zeros(B, H, N, dk, dtype=dtype),
            torch.zeros(B, H, N, dv, dtype=dtype))


def _state(B=1, H=2, dk=16, n=3, extra=0):
    return torch.zeros(B * H * ops.tt_state_floats(dk, 64, n) + extra)


def test_prefill_output_buffers(guard):
    Q, K, V = _qkv()
    with pytest.raises(ValueError, match="O must be float32"):
        ops.tt_prefill(Q, K, V, 3, O=torch.zeros(1, 2, 10, 64, dtype=torch.bfloat16), states=_state())
    with pytest.raises(ValueError, match="O must hold 1280"):
        ops.tt_prefill(Q, K, V, 3, O=torch.zeros(1, 2, 9, 64), states=_state())
    with pytest.raises(ValueError, match="states must hold"):
        ops.tt_prefill(Q, K, V, 3, O=torch.zeros(1, 2, 10, 64), states=_state(extra=-1))
    with pytest.raises(ValueError, match="states must hold"):
        ops.tt_prefill(Q, K, V, 3, O=torch.zeros(1, 2, 10, 64), states=_state(n=2))
    with pytest.raises(ValueError, match="must be contiguous"):
        ops.tt_prefill(Q, K, V, 3, O=torch.zeros(1, 2, 64, 10).transpose(2, 3), states=_state())


def test_prefill_inputs(guard):
    Q, K, V = _qkv()
    with pytest.raises(ValueError, match="share a dtype"):
        ops.tt_prefill(Q, K, V.float(), 3)
    with pytest.raises(ValueError, match="shape mismatch"):
        ops.tt_prefill(Q, K[:, :, :9], V, 3)
    with pytest.raises(ValueError, match="shape mismatch"):
        ops.tt_prefill(Q, K, V[:, :1], 3)
    with pytest.raises(ValueError, match="4-D"):
        ops.tt_prefill(Q[0], K[0], V[0], 3)
    with pytest.raises(ValueError, match="unsupported input dtype"):
        ops.tt_prefill(Q.half(), K.half(), V.half(), 3)


def test_prefill_from_and_unnormalized(guard):
    Q, K, V = _qkv()
    O, S = torch.zeros(1, 2, 10, 64), _state()
    with pytest.raises(ValueError, match="states_in must hold"):
        ops.tt_prefill_from(Q, K, V, _state(extra=5), 3, O=O, states=S)
    with pytest.raises(ValueError, match="states_in must be float32"):
        ops.tt_prefill_from(Q, K, V, _state().double(), 3, O=O, states=S)
    with pytest.raises(ValueError, match="states_in is None"):
        ops.tt_prefill_from(Q, K, V, None, 3, O=O, states=S)
    with pytest.raises(ValueError, match="den must hold 20"):
        ops.tt_prefill_from_unnormalized(Q, K, V, None, 3, num=O, den=torch.zeros(1, 2, 9), states=S)
    with pytest.raises(ValueError, match="states_in must hold"):
        ops.tt_prefill_normed(Q, K, V, 3, 1.0, states_in=_state(extra=1), O=O, states=S)


def test_decode_buffers(guard):
    q, k, v = torch.zeros(2, 3, 16), torch.zeros(2, 3, 16), torch.zeros(2, 3, 64)
    S = torch.zeros(6 * ops.tt_state_floats(16, 64, 3))
    with pytest.raises(ValueError, match="states must hold"):
        ops.tt_decode_step(q, k, v, S[:-1], 3)
    with pytest.raises(ValueError, match="states must hold"):
        ops.tt_decode_step(q, k, v, S, 2)
    with pytest.raises(ValueError, match="o must hold"):
        ops.tt_decode_step(q, k, v, S, 3, o=torch.zeros(2, 3, 63))
    with pytest.raises(ValueError, match="o must be float32"):
        ops.tt_decode_step(q, k, v, S, 3, o=torch.zeros(2, 3, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="share a dtype"):
        ops.tt_decode_step(q, k.bfloat16(), v, S, 3)
    with pytest.raises(ValueError, match="shape mismatch"):
        ops.tt_decode_step(q, k[:1], v, S, 3)
    with pytest.raises(ValueError, match="states must hold"):
        ops.tt_decode_step_normed(q, k, v, S[:10], 3, 1.0)


def test_merge_and_feature_map_buffers(guard):
    a, b = torch.zeros(100), torch.zeros(100)
    with pytest.raises(ValueError, match="b must hold 100"):
        ops.tt_state_merge(a, torch.zeros(99))
    with pytest.raises(ValueError, match="dst must hold 100"):
        ops.tt_state_merge(a, b, dst=torch.zeros(50))
    with pytest.raises(ValueError, match="dst must be float32"):
        ops.tt_state_merge(a, b, dst=torch.zeros(100, dtype=torch.float64))
    x = torch.zeros(5, 16)
    with pytest.raises(ValueError, match="out must hold 765"):
        ops.tt_feature_map(x, 3, True, out=torch.zeros(5, 152))


def test_softmax_buffers(guard):
    Q, K, V = _qkv()
    with pytest.raises(ValueError, match="O must hold"):
        ops.tt_softmax_prefill(Q, K, V, O=torch.zeros(10))
    q, k, v = torch.zeros(1, 2, 16), torch.zeros(1, 2, 16), torch.zeros(1, 2, 64)
    Kc, Vc = torch.zeros(1, 2, 100, 16), torch.zeros(1, 2, 100, 64)
    with pytest.raises(ValueError, match="do not match"):
        ops.tt_softmax_decode_step(q, k, v, Kc, Vc[:, :, :99], 5)
    with pytest.raises(ValueError, match="share a dtype"):
        ops.tt_softmax_decode_step(q, k, v, Kc.bfloat16(), Vc, 5)
    with pytest.raises(ValueError, match="workspace must hold"):
        ops.tt_softmax_decode_step(q, k, v, Kc, Vc, 5, workspace=torch.zeros(3, dtype=torch.uint8))


def test_device_check_comes_last(guard):
    """Well-formed host tensors get as far as the device check."""
    Q, K, V = _qkv()
    with pytest.raises(ValueError, match="must be a device tensor"):
        ops.tt_prefill(Q, K, V, 3, O=torch.zeros(1, 2, 10, 64), states=_state())
