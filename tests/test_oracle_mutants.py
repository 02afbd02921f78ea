"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each: the pins must be able to fail."""
import math

import numpy as np
import pytest

import oracle.taylor_oracle as orc
import pins
from taylor_recurrent_states_amd import workloads as wl

_orig_taylor = orc.taylor_kernel
_orig_feat = orc.feature_map
_orig_weights = orc.multinomial_weights
_orig_readout = orc._readout


def _taylor_dropped_term(x, n):
    return _orig_taylor(x, max(n - 1, 1)) if n > 1 else _orig_taylor(x, n)


def _taylor_wrong_factorial(x, n):
    x = np.asarray(x, dtype=np.float64)
    return sum(x ** m / max(m, 1) for m in range(n))


def _taylor_wrong_sign(x, n):
    x = np.asarray(x, dtype=np.float64)
    return sum((-x) ** m / math.factorial(m) if m == 1 else x ** m / math.factorial(m) for m in range(n))


def _weights_none(d, n):
    return np.ones_like(_orig_weights(d, n))


def _weights_mfact(d, n):
    # m!/alpha! instead of 1/alpha!: the multinomial count without the Taylor 1/m!
    w, r = _orig_weights(d, n).copy(), 0
    for m, width in enumerate(orc.block_widths(d, n)):
        w[r:r + width] *= math.factorial(m)
        r += width
    return w


def _feat_index_flip(X, n, weighted):
    X = np.asarray(X, dtype=np.float64)
    return _orig_feat(X[..., ::-1], n, weighted) if X.shape[-1] > 1 else _orig_feat(X, n, weighted)


def _feat_key_side_weighted(X, n, weighted):
    return _orig_feat(X, n, True)


def _readout_den_dropped_row0(phi, S):
    num = phi @ S[..., :-1]
    den = phi @ S[..., -1] - phi[..., 0] * S[..., 0, -1] + 1.0
    return num / den[..., None]


def _quadratic_exclusive(Q, K, V, n):
    Qh, lead = orc._heads(Q)
    Kh, _ = orc._heads(K)
    Vh, _ = orc._heads(V)
    N = Qh.shape[1]
    mask = np.tril(np.ones((N, N), dtype=bool), k=-1)
    mask[0, 0] = True
    out = np.empty(Vh.shape)
    for h in range(Qh.shape[0]):
        P = np.where(mask, orc.taylor_kernel(Qh[h] @ Kh[h].T, n), 0.0)
        out[h] = (P @ Vh[h]) / P.sum(axis=1, keepdims=True)
    return out.reshape(lead + Vh.shape[1:])


def _quadratic_transposed(Q, K, V, n):
    Qh, lead = orc._heads(Q)
    Kh, _ = orc._heads(K)
    Vh, _ = orc._heads(V)
    N = Qh.shape[1]
    mask = np.tril(np.ones((N, N), dtype=bool))
    out = np.empty(Vh.shape)
    for h in range(Qh.shape[0]):
        P = np.where(mask, orc.taylor_kernel(Kh[h] @ Qh[h].T, n), 0.0)
        out[h] = (P @ Vh[h]) / P.sum(axis=1, keepdims=True)
    return out.reshape(lead + Vh.shape[1:])


_orig_decode = orc.decode_step


def _decode_readout_first(q, k, v, S, n):
    o_old, _ = _orig_decode(q, np.zeros_like(np.asarray(k, dtype=np.float64)),
                            np.zeros_like(np.asarray(v, dtype=np.float64)), S, 1)
    _, S_new = _orig_decode(q, k, v, S, n)
    phi = orc.feature_map(q, n, True)
    num = np.einsum("...t,...tc->...c", phi, np.asarray(S)[..., :-1])
    den = np.einsum("...t,...t->...", phi, np.asarray(S)[..., -1])
    with np.errstate(invalid="ignore", divide="ignore"):
        return num / den[..., None], S_new


_orig_merge = orc.merge_states


def _merge_wrong(a, b):
    return np.asarray(a) + 0.5 * np.asarray(b)


_orig_planes = orc.states_to_planes


def _planes_interleaved(S):
    return np.asarray(S).reshape(-1)


_orig_prefill_from = orc.prefill_from_states


def _prefill_from_den_without_states(Q, K, V, S0, n):
    # the carried-in states enter the numerator only
    S0 = np.array(S0, dtype=np.float64)
    S0[..., -1] = 0.0
    o, _ = _orig_prefill_from(Q, K, V, S0, n)
    return o, orc.states_definition(K, V, n) + np.asarray(S0)


def _prefill_from_exclusive_states(Q, K, V, S0, n):
    # returns only the new tokens' states
    o, S = _orig_prefill_from(Q, K, V, S0, n)
    return o, S - np.asarray(S0)


_orig_softmax_rows = orc.softmax_rows


def _softmax_rows_exclusive(q_rows, K, V, rows):
    # the current key is left out (row 0 keeps its only key)
    out = []
    for r, i in enumerate(rows):
        j = max(i, 1)
        out.append(_orig_softmax_rows(q_rows[r:r + 1], np.asarray(K)[:j], np.asarray(V)[:j], [j - 1])[0])
    return np.stack(out)


def _softmax_rows_no_max(q_rows, K, V, rows):
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    out = []
    for r, i in enumerate(rows):
        p = np.exp(np.float32(K[: i + 1] @ np.asarray(q_rows[r])))  # no max subtracted, fp32 exp overflows
        out.append((p @ V[: i + 1]) / p.sum())
    return np.array(out)


_orig_normalize = orc.normalize_rows
_orig_round = orc.round_to_dtype


def _normalize_no_sqrt(X, scale=1.0):
    X = np.asarray(X, dtype=np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return X * (float(scale) / np.sum(X * X, axis=-1, keepdims=True))


def _normalize_inverted_temperature(X, scale=1.0):
    return _orig_normalize(X, 1.0 / float(scale))


def _round_via_f32(X, dtype):
    # rounds to fp32 first, then to bf16: two roundings
    if dtype != "bf16":
        return _orig_round(X, dtype)
    x32 = np.asarray(X, dtype=np.float64).astype(np.float32)
    return wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x32)).astype(np.float64)


def _round_truncating(X, dtype):
    if dtype != "bf16":
        return _orig_round(X, dtype)
    u = np.ascontiguousarray(X, dtype=np.float64).astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


_orig_numden = orc.prefill_from_numden
_orig_normalized_inputs = orc.normalized_inputs


def _normalized_inputs_tau_on_keys(Q, K, temperature, dtype):
    # the temperature also scales the keys
    return (orc.round_to_dtype(orc.normalize_rows(Q, temperature), dtype),
            orc.round_to_dtype(orc.normalize_rows(K, temperature), dtype))


def _numden_den_without_states(Q, K, V, S0, n):
    # the normaliser forgets the carried-in states' "+1" column
    num, den, S = _orig_numden(Q, K, V, S0, n)
    if S0 is None:
        return num, den, S
    phi = orc.feature_map(np.asarray(Q, dtype=np.float64), n, weighted=True)
    return num, den - phi @ np.asarray(S0, dtype=np.float64)[..., -1], S


MUTANTS = {
    "taylor_dropped_term": ("taylor_kernel", _taylor_dropped_term),
    "taylor_wrong_factorial": ("taylor_kernel", _taylor_wrong_factorial),
    "taylor_wrong_sign": ("taylor_kernel", _taylor_wrong_sign),
    "weights_missing": ("multinomial_weights", _weights_none),
    "weights_times_mfact": ("multinomial_weights", _weights_mfact),
    "feature_index_flip": ("feature_map", _feat_index_flip),
    "key_side_weighted": ("feature_map", _feat_key_side_weighted),
    "readout_den_row0": ("_readout", _readout_den_dropped_row0),
    "mask_exclusive": ("quadratic_attention", _quadratic_exclusive),
    "qk_transposed": ("quadratic_attention", _quadratic_transposed),
    "decode_readout_before_update": ("decode_step", _decode_readout_first),
    "merge_wrong": ("merge_states", _merge_wrong),
    "planes_interleaved": ("states_to_planes", _planes_interleaved),
    "prefill_from_den_without_states": ("prefill_from_states", _prefill_from_den_without_states),
    "prefill_from_exclusive_states": ("prefill_from_states", _prefill_from_exclusive_states),
    "numden_den_without_states": ("prefill_from_numden", _numden_den_without_states),
    "normalize_no_sqrt": ("normalize_rows", _normalize_no_sqrt),
    "normalize_inverted_temperature": ("normalize_rows", _normalize_inverted_temperature),
    "normalized_inputs_tau_on_keys": ("normalized_inputs", _normalized_inputs_tau_on_keys),
    "softmax_rows_exclusive": ("softmax_rows", _softmax_rows_exclusive),
    "softmax_rows_no_max": ("softmax_rows", _softmax_rows_no_max),
    "round_bf16_truncating": ("round_to_dtype", _round_truncating),
    "round_bf16_twice": ("round_to_dtype", _round_via_f32),
}

# cheap pins first; each mutant must make at least one of them fail
_PINS = [pins.pin_hand_example, pins.pin_kron_features, pins.pin_unit_identity,
         pins.pin_special_cases, pins.pin_decode_equals_recurrence,
         pins.pin_planes_layout, pins.pin_exact_rational, pins.pin_chunk_additivity,
         pins.pin_recurrent_vs_quadratic, pins.pin_softmax_library,
         pins.pin_softmax_convergence, pins.pin_prefill_from_states, pins.pin_prefill_from_numden,
         pins.pin_normalize_rows, pins.pin_normalized_inputs, pins.pin_round_to_dtype,
         pins.pin_softmax_rows]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in _PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, ZeroDivisionError, IndexError, KeyError):
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {name} passed every pin"
