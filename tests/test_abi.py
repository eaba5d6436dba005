"""The C-ABI library on the CPU: it loads, exports every function include/gdn.h
declares, and its host-side validation returns the documented status for each kind
of bad argument before anything reaches the GPU (these calls never launch)."""

import ctypes
import os
import re

import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from gated_deltanet_linear_causal_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, WORKSPACE, UNSUPPORTED, HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


NO_GPU = _no_gpu()

pytestmark = pytest.mark.skipif(not os.path.exists(gdn.library_path()), reason="libgdn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert set(names) >= {"gdn_conv_update", "gdn_recurrent_step", "gdn_decode_layer", "gdn_sequence",
                          "gdn_sequence_workspace_bytes", "gdn_status_string", "gdn_abi_version"}
    lib = ctypes.CDLL(gdn.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    for code in gdn.STATUS:
        assert gdn.gdn_status_string(code)
    assert gdn.gdn_status_string(12345) == "unknown status"
    assert gdn.gdn_abi_version() >> 16 == 1


def qwen(batch=4, **kw):
    args = dict(batch=batch, num_k_heads=16, num_v_heads=32, head_k_dim=128, head_v_dim=128)
    args.update(kw)
    return gdn.make_shape(**args)


class Fake:
    """Distinct, aligned, non-overlapping fake device addresses (never dereferenced)."""

    next = 1 << 40  # shared by all instances: addresses never repeat within a run

    def __call__(self, nbytes=1 << 32):
        p = Fake.next
        Fake.next += (nbytes + 4095) // 4096 * 4096 + (1 << 30)
        return ctypes.c_void_p(p)


def decode_args(shape, **override):
    f = Fake()
    names = ["conv1d_state", "state", "qkv", "conv1d_weight", "dt_raw", "b_raw", "z", "A_log", "dt_bias",
             "norm_weight", "out"]
    args = {n: f() for n in names}
    args.update(override)
    return [args[n] for n in names]


def call_decode(shape, **override):
    return gdn.library().gdn_decode_layer(ctypes.byref(shape), *decode_args(shape, **override), None)


def call_sequence(shape, T, ws=None, ws_bytes=0, **override):
    f = Fake()
    names = ["conv1d_state", "state", "qkv", "conv1d_weight", "dt_raw", "b_raw", "z", "A_log", "dt_bias",
             "norm_weight", "out"]
    args = {n: f() for n in names}
    args.update(override)
    return gdn.library().gdn_sequence(ctypes.byref(shape), T, *[args[n] for n in names], ws,
                                      ctypes.c_size_t(ws_bytes), None)


def test_null_shape_and_pointers():
    lib = gdn.library()
    assert lib.gdn_decode_layer(None, *decode_args(None), None) == NULL
    s = qwen()
    for i in range(11):
        args = decode_args(s)
        args[i] = None
        assert lib.gdn_decode_layer(ctypes.byref(s), *args, None) == NULL, i


def test_empty_batch_is_noop_with_null_pointers():
    s = qwen(batch=0)
    lib = gdn.library()
    assert lib.gdn_decode_layer(ctypes.byref(s), *([None] * 11), None) == OK
    assert lib.gdn_conv_update(ctypes.byref(s), None, None, None, None, None) == OK
    assert lib.gdn_recurrent_step(ctypes.byref(s), *([None] * 7), None) == OK
    assert call_sequence(qwen(), 0, **{n: None for n in ["conv1d_state", "state", "qkv"]}) == OK


@pytest.mark.parametrize("field,value,status", [
    ("batch", -1, SHAPE), ("num_k_heads", 0, SHAPE), ("num_v_heads", 0, SHAPE), ("num_v_heads", 33, SHAPE),
    ("head_k_dim", 0, SHAPE), ("conv_kernel", 1, SHAPE), ("conv_kernel", 9, SHAPE),
    ("l2_eps", -1.0, SHAPE), ("rms_eps", float("nan"), SHAPE), ("l2_eps", float("inf"), SHAPE),
    ("act_dtype", 7, DTYPE), ("out_dtype", -1, DTYPE),
    ("head_k_dim", 96, UNSUPPORTED), ("head_v_dim", 64, UNSUPPORTED), ("head_k_dim", 256, UNSUPPORTED),
])
def test_bad_shape_fields(field, value, status):
    s = qwen()
    if field in ("head_k_dim",) and value in (96, 256):
        s.head_v_dim = value
    setattr(s, field, value)
    assert call_decode(s) == status
    assert gdn.gdn_sequence_workspace_bytes(s, 4) == ctypes.c_size_t(-1).value


def test_too_many_v_heads_per_k_head():
    s = qwen(num_k_heads=1, num_v_heads=128)
    assert call_decode(s) == UNSUPPORTED


def test_grid_overflow():
    s = qwen(batch=2 ** 30)
    assert call_decode(s) == SHAPE


def test_misaligned():
    s = qwen()
    f = Fake()
    assert call_decode(s, state=ctypes.c_void_p(f().value + 4)) == ALIGN
    assert call_decode(s, qkv=ctypes.c_void_p(f().value + 2)) == ALIGN
    base = f().value
    assert call_decode(s, dt_raw=ctypes.c_void_p(base + 1)) == ALIGN


@pytest.mark.skipif(NO_GPU is False, reason="these calls pass validation and would launch on fake pointers")
def test_valid_calls_reach_the_launch():
    """Arguments that validation must accept reach the launch, which fails with
    GDN_ERR_HIP on a host without a GPU (the pointers are fake)."""
    s = qwen()
    f = Fake()
    # dt_raw only needs element alignment (bf16: 2 bytes)
    assert call_decode(s, dt_raw=ctypes.c_void_p(f().value + 2)) == HIP
    # read-only inputs may share memory
    r = f()
    assert call_decode(s, A_log=r, dt_bias=r) == HIP


def test_aliasing():
    s = qwen()
    f = Fake()
    p = f()
    assert call_decode(s, state=p, out=p) == ALIAS
    q = f()
    # out overlapping the tail of z
    z_bytes = s.batch * s.num_v_heads * s.head_v_dim * 2
    assert call_decode(s, z=q, out=ctypes.c_void_p(q.value + z_bytes - 16)) == ALIAS


def test_sequence_validation():
    s = qwen()
    assert call_sequence(s, -1) == SHAPE
    assert gdn.gdn_sequence_workspace_bytes(s, 16) == 0
    assert gdn.gdn_sequence_workspace_bytes(s, -1) == ctypes.c_size_t(-1).value
    f = Fake()
    assert call_sequence(s, 3, out=ctypes.c_void_p(f().value + 8)) == ALIGN


def _row_bytes(s):
    C = 2 * s.num_k_heads * s.head_k_dim + s.num_v_heads * s.head_v_dim
    ea = 2 if s.act_dtype == 1 else 4
    eo = 2 if s.out_dtype == 1 else 4
    return max(C * ea, s.num_v_heads * s.head_v_dim * max(ea, eo))


def test_sequence_rejects_buffers_past_2_62_bytes():
    """B x T times a token's largest row (qkv, z or out) above 2^62 bytes is a shape
    error (no buffer size may wrap in 64 bits); at exactly 2^62 the shape passes and the
    call goes on to the buffer checks (here: the fake buffers overlap)."""
    SIZE_MAX = ctypes.c_size_t(-1).value
    big = qwen(batch=1 << 18)                     # row = 16 KiB (fp32 out)
    assert _row_bytes(big) == 1 << 14
    T = (1 << 30) + 1                             # 2^18 x T x 2^14 > 2^62
    assert gdn.gdn_sequence_workspace_bytes(big, T) == SIZE_MAX
    assert call_sequence(big, T) == SHAPE
    edge = qwen(batch=1 << 17)
    T = (1 << 31) - 1                             # 2^17 x T x 2^14 < 2^62
    assert gdn.gdn_sequence_workspace_bytes(edge, T) == 0
    assert call_sequence(edge, T) == ALIAS
    huge = qwen(batch=(1 << 27) - 1, num_k_heads=16)  # B x H_k just below 2^31
    assert gdn.gdn_sequence_workspace_bytes(huge, (1 << 31) - 1) == SIZE_MAX
    assert call_sequence(huge, (1 << 31) - 1) == SHAPE


@settings(max_examples=300, deadline=None)
@given(batch=st.integers(0, (1 << 31) - 1), hk=st.integers(1, 64), g=st.sampled_from([1, 2, 4]),
       d=st.sampled_from([32, 64, 128]), T=st.integers(0, (1 << 31) - 1), act=st.sampled_from([0, 1]),
       out=st.sampled_from([0, 1]))
def test_sequence_size_rule_matches_the_definition(batch, hk, g, d, T, act, out):
    """The workspace query (host-only, never launches) accepts exactly the shapes whose
    grid fits and whose B x T x largest token row is at most 2^62 bytes."""
    s = gdn.make_shape(batch, hk, hk * g, d, d, 4, 1e-6, 1e-6, act, out)
    grid_ok = batch * hk <= (1 << 31) - 1
    ok = grid_ok and batch * T * _row_bytes(s) <= 1 << 62
    assert (gdn.gdn_sequence_workspace_bytes(s, T) == 0) == ok


def test_header_mentions_every_status():
    text = open(HEADER).read()
    for name in gdn.STATUS.values():
        assert name in text


def test_pooled_validation():
    s = qwen()
    f = Fake()
    args = [f() for _ in range(12)]  # slots, two pools, qkv, taps, dt, b, z, A_log, dt_bias, norm_w, out
    lib = gdn.library()
    assert lib.gdn_decode_layer_pooled(ctypes.byref(s), -1, *args, None) == SHAPE
    bad = list(args)
    bad[0] = ctypes.c_void_p(args[0].value + 2)  # slots must be 4-byte aligned
    assert lib.gdn_decode_layer_pooled(ctypes.byref(s), 8, *bad, None) == ALIGN
    bad = list(args)
    bad[1] = None
    assert lib.gdn_decode_layer_pooled(ctypes.byref(s), 8, *bad, None) == NULL
    # an empty pool needs no state pointers and launches nothing
    bad = list(args)
    bad[1] = bad[2] = None
    assert lib.gdn_decode_layer_pooled(ctypes.byref(s), 0, *bad, None) == OK


def call_verify(shape, T, trail=None, trail_bytes=None, **override):
    f = Fake()
    names = ["conv1d_state", "state", "qkv", "conv1d_weight", "dt_raw", "b_raw", "z", "A_log", "dt_bias",
             "norm_weight", "out"]
    args = {n: f() for n in names}
    args.update(override)
    if trail is None:
        trail = f()
    if trail_bytes is None:
        trail_bytes = gdn.gdn_verify_trail_bytes(shape, T)
    return gdn.library().gdn_decode_verify(ctypes.byref(shape), T, *[args[n] for n in names], trail,
                                           ctypes.c_size_t(trail_bytes), None)


def call_commit(shape, T, trail=None, trail_bytes=None, **override):
    f = Fake()
    names = ["accepted", "conv1d_state", "state", "qkv"]
    args = {n: f() for n in names}
    args.update(override)
    if trail is None:
        trail = f()
    if trail_bytes is None:
        trail_bytes = gdn.gdn_verify_trail_bytes(shape, T)
    return gdn.library().gdn_decode_commit(ctypes.byref(shape), T, *[args[n] for n in names], trail,
                                           ctypes.c_size_t(trail_bytes), None)


def test_verify_trail_bytes():
    s = qwen(batch=3)
    for T in range(0, gdn.GDN_MAX_VERIFY_TOKENS + 1):
        # delta [B][T][Hv][d] + unit k [B][T][Hk][d] + alpha [B][T][Hv], fp32
        assert gdn.gdn_verify_trail_bytes(s, T) == 4 * 3 * T * (32 * 128 + 16 * 128 + 32)
    for T in (-1, gdn.GDN_MAX_VERIFY_TOKENS + 1):
        assert gdn.gdn_verify_trail_bytes(s, T) == ctypes.c_size_t(-1).value


def test_verify_commit_validation():
    s = qwen()
    for T in (-1, gdn.GDN_MAX_VERIFY_TOKENS + 1):
        assert call_verify(s, T, trail_bytes=0) == SHAPE
        assert call_commit(s, T, trail_bytes=0) == SHAPE
    # no tokens, or no sequences: nothing to do, pointers may be NULL
    assert call_verify(s, 0, trail=None, **{n: None for n in ["conv1d_state", "state", "qkv", "out"]}) == OK
    assert call_commit(qwen(batch=0), 4, **{n: None for n in ["accepted", "conv1d_state", "state", "qkv"]}) == OK
    need = gdn.gdn_verify_trail_bytes(s, 4)
    assert call_verify(s, 4, trail_bytes=need - 4) == WORKSPACE
    assert call_commit(s, 4, trail_bytes=need - 4) == WORKSPACE
    assert call_verify(s, 4, out=None) == NULL
    assert call_commit(s, 4, accepted=None) == NULL
    f = Fake()
    assert call_commit(s, 4, accepted=ctypes.c_void_p(f().value + 2)) == ALIGN
    assert call_verify(s, 4, trail=ctypes.c_void_p(f().value + 8)) == ALIGN
    # the trail is written by verify and may not overlap the output; commit writes the states
    p = f()
    assert call_verify(s, 4, trail=p, out=p) == ALIAS
    q = f()
    assert call_commit(s, 4, trail=q, state=q) == ALIAS


@pytest.mark.skipif(NO_GPU is False, reason="these calls pass validation and would launch on fake pointers")
def test_verify_reads_states_only():
    """gdn_decode_verify only reads the states, so they may share memory with other
    read-only inputs: validation accepts it (the launch then fails on a host without a
    GPU, the pointers being fake)."""
    r = Fake()()
    assert call_verify(qwen(), 4, conv1d_state=r, qkv=r) == HIP


def call_in_proj(shape, hidden, **override):
    f = Fake()
    names = ["x_norm", "w_qkv", "w_z", "w_a", "w_b", "qkv", "z", "dt_raw", "b_raw"]
    args = {n: f() for n in names}
    args.update(override)
    return gdn.library().gdn_in_proj(ctypes.byref(shape), hidden, *[args[n] for n in names], None)


def call_out_proj(shape, hidden, **override):
    f = Fake()
    names = ["gated", "w_out", "y"]
    args = {n: f() for n in names}
    args.update(override)
    return gdn.library().gdn_out_proj(ctypes.byref(shape), hidden, *[args[n] for n in names], None)


def test_projection_validation():
    s = qwen()
    assert call_in_proj(s, 0) == SHAPE
    assert call_out_proj(s, -64) == SHAPE
    assert call_in_proj(s, 2000) == UNSUPPORTED      # in_proj contracts over hidden: a multiple of 64
    assert call_in_proj(qwen(act_dtype="f32"), 2048) == UNSUPPORTED
    assert call_out_proj(qwen(act_dtype="f32"), 2048) == UNSUPPORTED
    # out_proj contracts over H_v * d_v, which must also be a multiple of 64
    assert call_out_proj(qwen(num_k_heads=1, num_v_heads=1, head_k_dim=32, head_v_dim=32), 2048) == UNSUPPORTED
    assert call_in_proj(s, 2048, w_z=None) == NULL
    assert call_out_proj(s, 2048, y=None) == NULL
    assert call_in_proj(qwen(batch=0), 2048, **{n: None for n in ["x_norm", "qkv", "z", "dt_raw", "b_raw"]}) == OK
    f = Fake()
    assert call_in_proj(s, 2048, x_norm=ctypes.c_void_p(f().value + 8)) == ALIGN
    assert call_in_proj(s, 2048, w_a=ctypes.c_void_p(f().value + 2)) == ALIGN
    p = f()
    assert call_in_proj(s, 2048, qkv=p, z=p) == ALIAS
    q = f()
    assert call_out_proj(s, 2048, gated=q, y=q) == ALIAS
    assert call_in_proj(qwen(batch=65535 * 32 + 1), 2048) == SHAPE


def call_debug(shape, **override):
    f = Fake()
    names = ["conv1d_state", "state", "qkv", "conv1d_weight", "dt_raw", "b_raw", "z", "A_log", "dt_bias",
             "norm_weight", "out", "qkv_act", "alpha", "beta", "y", "y_norm"]
    args = {n: f() for n in names}
    args.update(override)
    return gdn.library().gdn_decode_layer_debug(ctypes.byref(shape), *[args[n] for n in names], None)


def test_debug_taps_validation():
    """gdn_decode_layer_debug: the decode step's checks, plus its optional taps: a null
    tap is allowed, a misaligned y / y_norm tap or a tap overlapping another buffer is
    rejected before any launch."""
    s = qwen()
    f = Fake()
    assert call_debug(s, state=None) == NULL
    assert call_debug(s, y=ctypes.c_void_p(f().value + 4)) == ALIGN
    assert call_debug(s, y_norm=ctypes.c_void_p(f().value + 8)) == ALIGN
    out = f()
    assert call_debug(s, out=out, y=out) == ALIAS
    assert call_debug(s, alpha=ctypes.c_void_p(f().value + 2)) == ALIGN
    assert call_debug(qwen(batch=0), **{n: None for n in ["conv1d_state", "state", "qkv", "out", "y"]}) == OK
    if NO_GPU:  # every tap null: validation passes and the (fake) launch fails
        assert call_debug(s, qkv_act=None, alpha=None, beta=None, y=None, y_norm=None) == HIP
