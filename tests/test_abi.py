"""The C-ABI library loads, exports every declared symbol, and validates
arguments on the host (no kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest

from taylor_recurrent_states_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "taylor_states.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tt_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = ops.lib()
    declared = _declared()
    assert set(declared) == set(ops.EXPORTED), declared
    for name in declared:
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_state_sizes():
    assert ops.tt_state_rows(16, 3) == 153
    assert ops.tt_state_floats(16, 64, 3) == 9945
    assert ops.tt_state_floats(16, 64, 5) == 314925
    assert ops.tt_state_floats(64, 64, 3) == 139425
    assert ops.tt_state_rows(16, 1) == 1
    assert ops.tt_state_rows(0, 3) == 0
    assert ops.tt_state_rows(16, 0) == 0
    assert ops.tt_state_floats(16, 0, 3) == 0
    assert ops.tt_state_rows(1 << 30, 40) == 0  # overflow -> 0


def test_workspace_query_and_errors():
    assert ops.tt_prefill_workspace_bytes(4, 8, 8192, 16, 64, 3, 64) >= 0
    with pytest.raises(ops.TTError) as e:
        ops.tt_prefill_workspace_bytes(1, 1, 0, 16, 64, 3, 64)
    assert e.value.code == ops.TT_ERR_INVALID_ARG
    with pytest.raises(ops.TTError) as e:
        ops.tt_prefill_workspace_bytes(1, 1, 16, 16, 48, 3, 64)
    assert e.value.code == ops.TT_ERR_UNSUPPORTED
    with pytest.raises(ops.TTError) as e:
        ops.tt_prefill_workspace_bytes(1, 1, 16, 64, 64, 6, 64)
    assert e.value.code == ops.TT_ERR_UNSUPPORTED


def test_widest_shapes_plan_the_streamed_path():
    """dk = 32 and 64 with four and five terms: one span state of the padded
    rows (128-row groups) per (head, span of 1,024 tokens), for both dtypes
    (both run the fp32 streamed kernels); other chunk lengths are refused."""
    for dk, n, W in ((32, 4, 6545), (32, 5, 58905), (64, 4, 47905), (64, 5, 814385)):
        assert ops.tt_state_rows(dk, n) == W
        wp = (W + 127) // 128 * 128
        for dt in ("f32", "bf16"):
            assert ops.tt_prefill_workspace_bytes_dtype(2, 3, 1100, dk, 64, n, 64, dt) == 2 * 3 * 2 * wp * 65 * 4
        for chunk in (16, 32, 128):
            with pytest.raises(ops.TTError) as e:
                ops.tt_prefill_workspace_bytes(1, 1, 100, dk, 64, n, chunk)
            assert e.value.code == ops.TT_ERR_UNSUPPORTED


def test_head_groups_need_one_heads_share_of_the_workspace():
    """A streamed plan takes a workspace of at least one head's share (it
    then runs the heads in groups), with or without the normalisation; the
    other plans take the whole workspace.  Smaller ones are refused before
    anything is launched."""
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)
    ws = ctypes.c_void_p(0x100000)
    need = ops.tt_prefill_workspace_bytes_dtype(1, 3, 1100, 64, 64, 3, 64, "bf16")
    per_head = need // 3
    assert per_head * 3 == need
    rc = L.tt_prefill(fake, fake, fake, 1, 1, 3, 1100, 64, 64, 3, 64, fake, fake, ws, per_head - 256, None)
    assert rc == ops.TT_ERR_WORKSPACE and "per head" in ops.tt_last_error()
    need = ops.tt_prefill_workspace_bytes_dtype(1, 3, 1100, 16, 64, 3, 32, "f32")  # the chunk-32 sweep
    rc = L.tt_prefill(fake, fake, fake, 0, 1, 3, 1100, 16, 64, 3, 32, fake, fake, ws, need - 256, None)
    assert rc == ops.TT_ERR_WORKSPACE and "per head" not in ops.tt_last_error()
    # the normalised prefill: one head's share of its workspace (the query at B = H = 1), not less
    w1 = ops.tt_prefill_normed_workspace_bytes(1, 1, 1100, 64, 64, 3)
    rc = L.tt_prefill_normed(fake, fake, fake, 1, 1, 3, 1100, 64, 64, 3, 64, ctypes.c_float(1.0), None, fake, fake,
                             ws, w1 // 2, None)
    assert rc == ops.TT_ERR_WORKSPACE and "per head" in ops.tt_last_error()
    rc = L.tt_prefill_normed(ctypes.c_void_p(0x1002), fake, fake, 1, 1, 3, 1100, 64, 64, 3, 64, ctypes.c_float(1.0),
                             None, fake, fake, ws, w1, None)
    assert rc == ops.TT_ERR_INVALID_ARG and "aligned" in ops.tt_last_error()
    # a sweep plan's normalised prefill takes its whole workspace
    rc = L.tt_prefill_normed(fake, fake, fake, 0, 1, 3, 1100, 16, 64, 3, 32, ctypes.c_float(1.0), None, fake, fake,
                             ws, 4096, None)
    assert rc == ops.TT_ERR_WORKSPACE and "per head" not in ops.tt_last_error()
    # one head's share passes the workspace check (a misaligned Q then stops the call)
    odd = ctypes.c_void_p(0x1002)
    for B, H, N, dk, n, dt in ((1, 5, 2100, 64, 3, "bf16"), (2, 2, 1500, 16, 5, "f32"), (1, 3, 1100, 32, 4, "bf16"),
                               (1, 3, 1100, 64, 5, "bf16"), (1, 3, 1100, 32, 3, "bf16")):
        need = ops.tt_prefill_workspace_bytes_dtype(B, H, N, dk, 64, n, 64, dt)
        assert need % (B * H) == 0
        code = 1 if dt == "bf16" else 0
        rc = L.tt_prefill(odd, fake, fake, code, B, H, N, dk, 64, n, 64, fake, fake, ws, need // (B * H), None)
        assert rc == ops.TT_ERR_INVALID_ARG and "aligned" in ops.tt_last_error(), (B, H, N, dk, n, dt)
    # tt_prefill_noalloc: one head's share must fit its array
    assert ops.tt_prefill_workspace_bytes_dtype(1, 16, 8192, 16, 64, 5, 32, "f32") > ops.TT_NOALLOC_SCRATCH_BYTES
    rc = L.tt_prefill_noalloc(fake, fake, fake, 0, 1, 16, 8192, 16, 64, 5, 32, fake, fake, None)
    assert rc == ops.TT_ERR_WORKSPACE and "noalloc" in ops.tt_last_error()


def test_entry_points_reject_bad_arguments_without_launching():
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    rc = L.tt_decode_step(None, fake, fake, 0, 1, 1, 16, 64, 3, fake, fake, None)
    assert rc == ops.TT_ERR_INVALID_ARG and "NULL" in ops.tt_last_error()
    rc = L.tt_decode_step(fake, fake, fake, 7, 1, 1, 16, 64, 3, fake, fake, None)
    assert rc == ops.TT_ERR_INVALID_ARG
    rc = L.tt_decode_step(fake, fake, fake, 0, 1, 1, 16, 64, 9, fake, fake, None)
    assert rc == ops.TT_ERR_UNSUPPORTED
    rc = L.tt_decode_step(fake, fake, fake, 0, 0, 1, 16, 64, 3, fake, fake, None)
    assert rc == ops.TT_ERR_INVALID_ARG
    rc = L.tt_prefill(fake, fake, fake, 1, 1, 1, 100, 16, 64, 3, 64, fake, fake, None, 0, None)
    need = ops.tt_prefill_workspace_bytes(1, 1, 100, 16, 64, 3, 64)
    if need > 0:
        assert rc == ops.TT_ERR_WORKSPACE
    rc = L.tt_prefill(fake, fake, fake, 1, 1, 1, 100, 16, 64, 3, 48, fake, fake, fake, 1 << 30, None)
    assert rc == ops.TT_ERR_UNSUPPORTED
    ws = ctypes.c_void_p(0x100000)
    rc = L.tt_prefill_from(fake, fake, fake, 1, 1, 1, 100, 16, 64, 3, 64, None, fake, fake, ws, 1 << 30, None)
    assert rc == ops.TT_ERR_INVALID_ARG and "states_in" in ops.tt_last_error()
    nbytes = ops.tt_state_floats(16, 64, 3) * 4
    # states_in overlapping states without being the same buffer
    s_out, s_in = 0x40000000, 0x40000000 + 64
    rc = L.tt_prefill_from(fake, fake, fake, 1, 1, 1, 100, 16, 64, 3, 64, ctypes.c_void_p(s_in), fake,
                           ctypes.c_void_p(s_out), ws, 1 << 30, None)
    assert rc == ops.TT_ERR_INVALID_ARG and "overlap" in ops.tt_last_error()
    # states_in overlapping the workspace
    rc = L.tt_prefill_from(fake, fake, fake, 1, 1, 1, 100, 16, 64, 3, 64, ctypes.c_void_p(0x100000 + 4096), fake,
                           ctypes.c_void_p(s_out), ws, 1 << 30, None)
    assert rc == ops.TT_ERR_INVALID_ARG and "overlap" in ops.tt_last_error()
    assert nbytes > 64
    rc = L.tt_state_merge(None, fake, fake, 4, None)
    assert rc == ops.TT_ERR_INVALID_ARG
    assert L.tt_state_merge(None, None, None, 0, None) == ops.TT_OK
    rc = L.tt_feature_map(fake, 0, 4, 16, 3, 2, fake, None)
    assert rc == ops.TT_ERR_INVALID_ARG
    assert L.tt_feature_map(None, 0, 0, 16, 3, 0, None, None) == ops.TT_OK


def test_unnormalized_prefill_rejects_bad_arguments_without_launching():
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)
    args = (fake, fake, fake, 0, 1, 1, 64, 16, 64, 3, 64)
    # den NULL
    rc = L.tt_prefill_from_unnormalized(*args, None, ctypes.c_void_p(0x100000), None, fake, fake, 1 << 30, None)
    assert rc == ops.TT_ERR_INVALID_ARG and "den" in ops.tt_last_error()
    # den not 4-byte aligned
    rc = L.tt_prefill_from_unnormalized(*args, None, ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200002), fake, fake,
                                        1 << 30, None)
    assert rc == ops.TT_ERR_INVALID_ARG
    # den overlapping the numerators
    rc = L.tt_prefill_from_unnormalized(*args, None, ctypes.c_void_p(0x100000), ctypes.c_void_p(0x100010), fake,
                                        ctypes.c_void_p(0x90000000), 1 << 30, None)
    assert rc == ops.TT_ERR_INVALID_ARG and "overlap" in ops.tt_last_error()


def test_normalised_entry_points_reject_bad_arguments_without_launching():
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)
    f = ctypes.c_float
    assert L.tt_normalize_rows(None, 0, 0, 16, f(1.0), None, None) == ops.TT_OK  # rows == 0: no-op
    assert L.tt_normalize_rows(None, 0, 4, 16, f(1.0), fake, None) == ops.TT_ERR_INVALID_ARG
    assert L.tt_normalize_rows(fake, 0, 4, 24, f(1.0), fake, None) == ops.TT_ERR_UNSUPPORTED
    assert L.tt_normalize_rows(fake, 3, 4, 16, f(1.0), fake, None) == ops.TT_ERR_INVALID_ARG
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert L.tt_normalize_rows(fake, 0, 4, 16, f(bad), fake, None) == ops.TT_ERR_INVALID_ARG
        assert "scale" in ops.tt_last_error()
    assert L.tt_normalize_rows(ctypes.c_void_p(0x1004), 0, 4, 16, f(1.0), fake, None) == ops.TT_ERR_INVALID_ARG
    # out overlapping x without being x
    assert L.tt_normalize_rows(fake, 0, 4, 16, f(1.0), ctypes.c_void_p(0x1010), None) == ops.TT_ERR_INVALID_ARG
    ws = ctypes.c_void_p(0x100000)
    need = ops.tt_prefill_normed_workspace_bytes(1, 1, 100, 16, 64, 3, 64)
    assert need > ops.tt_prefill_workspace_bytes(1, 1, 100, 16, 64, 3, 64) + 2 * 100 * 16 * 2
    rc = L.tt_prefill_normed(fake, fake, fake, 1, 1, 1, 100, 16, 64, 3, 64, f(1.0), None, fake, fake, ws, need - 1,
                             None)
    assert rc == ops.TT_ERR_WORKSPACE
    rc = L.tt_prefill_normed(fake, fake, fake, 1, 1, 1, 100, 16, 64, 3, 64, f(0.0), None, fake, fake, ws, need, None)
    assert rc == ops.TT_ERR_INVALID_ARG and "temperature" in ops.tt_last_error()
    rc = L.tt_decode_step_normed(fake, fake, fake, 0, 1, 1, 16, 64, 3, f(-2.0), fake, fake, None)
    assert rc == ops.TT_ERR_INVALID_ARG and "temperature" in ops.tt_last_error()
    rc = L.tt_decode_step_normed(None, fake, fake, 0, 1, 1, 16, 64, 3, f(1.0), fake, fake, None)
    assert rc == ops.TT_ERR_INVALID_ARG


def test_softmax_entry_points_reject_bad_arguments_without_launching():
    L = ops.lib()
    fake = ctypes.c_void_p(0x1000)
    rc = L.tt_softmax_prefill(fake, fake, fake, 0, 1, 1, 64, 16, 64, fake, None)
    assert rc == ops.TT_ERR_UNSUPPORTED and "bf16" in ops.tt_last_error()
    assert L.tt_softmax_prefill(fake, fake, fake, 1, 1, 1, 64, 24, 64, fake, None) == ops.TT_ERR_UNSUPPORTED
    assert L.tt_softmax_prefill(None, fake, fake, 1, 1, 1, 64, 16, 64, fake, None) == ops.TT_ERR_INVALID_ARG
    assert L.tt_softmax_prefill(fake, fake, fake, 1, 1, 1, 0, 16, 64, fake, None) == ops.TT_ERR_INVALID_ARG
    assert ops.tt_softmax_decode_workspace_bytes(2, 3, 0) == 2 * 3 * 66 * 4
    assert ops.tt_softmax_decode_workspace_bytes(2, 3, 2048) == 2 * 3 * 2 * 66 * 4
    ws = ctypes.c_void_p(0x100000)
    args = (fake, fake, fake, 0, 1, 1, 16, 64, fake, fake)
    assert L.tt_softmax_decode_step(*args, 5, 5, fake, ws, 1 << 20, None) == ops.TT_ERR_INVALID_ARG  # pos == cap
    assert L.tt_softmax_decode_step(*args, -1, 5, fake, ws, 1 << 20, None) == ops.TT_ERR_INVALID_ARG
    assert L.tt_softmax_decode_step(*args, 3, 5, fake, ws, 10, None) == ops.TT_ERR_WORKSPACE
    assert L.tt_softmax_decode_step(*args, 3, 5, fake, None, 0, None) == ops.TT_ERR_WORKSPACE
    bad = (fake, fake, fake, 0, 1, 1, 16, 64, ctypes.c_void_p(0x1008), fake)
    assert L.tt_softmax_decode_step(*bad, 3, 5, fake, ws, 1 << 20, None) == ops.TT_ERR_INVALID_ARG


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The package never imports the oracle and has no host compute path."""
    pkg = os.path.join(ROOT, "taylor_recurrent_states_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "taylor_oracle" not in text, f


def test_small_key_width_plans():
    """dk = 8 runs up to six terms (C(13, 5) = 1287 feature rows); its
    prefill takes fp32 inputs only, refused before anything is launched."""
    assert ops.tt_state_rows(8, 6) == 1287
    assert ops.tt_state_floats(8, 64, 6) == 1287 * 65
    assert ops.tt_prefill_workspace_bytes(1, 16, 4096, 8, 64, 6, 64) > 0
    with pytest.raises(ops.TTError) as e:
        ops.tt_prefill_workspace_bytes(1, 1, 16, 8, 64, 7, 64)
    assert e.value.code == ops.TT_ERR_UNSUPPORTED
    L = ops.lib()
    misaligned, fake = ctypes.c_void_p(0x1001), ctypes.c_void_p(0x1000)  # never reaches a launch
    rc = L.tt_prefill(misaligned, fake, fake, ops.TT_BF16, 1, 1, 100, 8, 64, 3, 64, fake, fake, fake, 1 << 30, None)
    assert rc == ops.TT_ERR_UNSUPPORTED and "fp32" in ops.tt_last_error()


def test_chunk_lengths_are_validated_before_launch():
    """chunk in {16, 32, 64, 128}; bf16 takes 32 or more; 128 runs the shapes
    whose tiles fit the LDS and refuses the others, all before any launch."""
    L = ops.lib()
    # Q misaligned: a shape the plan accepts fails the alignment check that
    # follows it (INVALID_ARG), so no call here can reach a launch
    misaligned, fake = ctypes.c_void_p(0x1001), ctypes.c_void_p(0x1000)

    def rc(dt, dk, n, chunk):
        return L.tt_prefill(misaligned, fake, fake, dt, 1, 1, 100, dk, 64, n, chunk, fake, fake, fake, 1 << 40, None)

    for chunk in (0, 8, 48, 96, 256):
        assert rc(ops.TT_F32, 16, 3, chunk) == ops.TT_ERR_UNSUPPORTED
    assert rc(ops.TT_BF16, 16, 3, 16) == ops.TT_ERR_UNSUPPORTED
    assert rc(ops.TT_BF16, 16, 3, 128) == ops.TT_ERR_INVALID_ARG
    assert rc(ops.TT_BF16, 64, 3, 128) == ops.TT_ERR_UNSUPPORTED
    assert rc(ops.TT_F32, 8, 6, 16) == ops.TT_ERR_INVALID_ARG
    for chunk in (16, 32, 64, 128):
        assert ops.tt_prefill_workspace_bytes(2, 4, 1000, 16, 64, 3, chunk) > 0


def test_workspace_query_per_dtype():
    """tt_prefill_workspace_bytes_dtype: the exact workspace of one input
    dtype, never more than the dtype-free query; the shapes whose two dtypes
    run different kernels differ."""
    for args in [(4, 8, 8192, 16, 64, 3, 64), (1, 16, 65536, 64, 64, 3, 64), (1, 16, 16384, 16, 64, 5, 64),
                 (2, 3, 1000, 32, 64, 3, 32), (1, 2, 100, 8, 64, 6, 64)]:
        both = ops.tt_prefill_workspace_bytes(*args)
        per = {}
        for dt in ("f32", "bf16"):
            try:
                per[dt] = ops.tt_prefill_workspace_bytes_dtype(*args, dtype=dt)
            except ops.TTError as e:
                assert e.code == ops.TT_ERR_UNSUPPORTED  # dk = 8 prefill is fp32 only
        assert per and max(per.values()) == both, (args, per, both)
    # wide keys: bf16 keeps octet rows (more padded rows than fp32's feature order)
    f = ops.tt_prefill_workspace_bytes_dtype(1, 16, 65536, 64, 64, 3, 64, "f32")
    b = ops.tt_prefill_workspace_bytes_dtype(1, 16, 65536, 64, 64, 3, 64, "bf16")
    assert f < b
    # order 5 at dk 16: both dtypes run the fp32 streamed kernels, one workspace
    f = ops.tt_prefill_workspace_bytes_dtype(1, 16, 16384, 16, 64, 5, 64, "f32")
    b = ops.tt_prefill_workspace_bytes_dtype(1, 16, 16384, 16, 64, 5, 64, "bf16")
    assert f == b
    with pytest.raises(ValueError):
        ops.tt_prefill_workspace_bytes_dtype(1, 1, 10, 16, 64, 3, 64, "f16")
    L = ops.lib()
    out = ctypes.c_size_t(0)
    assert L.tt_prefill_workspace_bytes_dtype(1, 1, 10, 16, 64, 3, 64, 7, ctypes.byref(out)) == ops.TT_ERR_INVALID_ARG
