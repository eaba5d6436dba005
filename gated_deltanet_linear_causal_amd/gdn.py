"""Python binding of libgdn.so (include/gdn.h), by ctypes.

Argument marshalling only: tensors become device pointers, the current torch stream
becomes the hipStream_t, and a nonzero status raises GdnError. Every step of the
computation runs in the library's HIP kernels; there is no other code path, and a
missing library raises at first use.

Before passing pointers, each tensor is checked to be a contiguous tensor on the GPU
with the dtype and at least the number of elements the shape implies, so that the
library never reads or writes past a tensor it was given. These checks cost about half
a microsecond per tensor; a caller that has checked its buffers once (a serving loop
over fixed buffers) may pass validate=False to skip them, and the library's own checks
(null pointers, alignment, aliasing, the shape) still run.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "GDN_F32", "GDN_BF16", "GdnError", "GdnShape", "make_shape", "library", "library_path",
    "gdn_conv_update", "gdn_recurrent_step", "gdn_decode_layer", "gdn_decode_layer_pooled", "gdn_sequence",
    "gdn_sequence_workspace_bytes", "gdn_verify_trail_bytes", "gdn_decode_verify", "gdn_decode_commit",
    "GDN_MAX_VERIFY_TOKENS", "gdn_in_proj", "gdn_out_proj", "gdn_status_string", "gdn_abi_version", "STATUS",
]

GDN_F32 = 0
GDN_BF16 = 1
GDN_MAX_VERIFY_TOKENS = 8

STATUS = {0: "GDN_OK", -1: "GDN_ERR_NULL", -2: "GDN_ERR_SHAPE", -3: "GDN_ERR_DTYPE",
          -4: "GDN_ERR_ALIGN", -5: "GDN_ERR_ALIAS", -6: "GDN_ERR_WORKSPACE",
          -7: "GDN_ERR_UNSUPPORTED", -8: "GDN_ERR_HIP"}

_PKG = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_PKG, "libgdn.so")


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, STATUS.get(status, status), gdn_status_string(status)))


class GdnShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_k_heads", ctypes.c_int32),
                ("num_v_heads", ctypes.c_int32), ("head_k_dim", ctypes.c_int32),
                ("head_v_dim", ctypes.c_int32), ("conv_kernel", ctypes.c_int32),
                ("l2_eps", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]

    @property
    def channels(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim


def make_shape(batch, num_k_heads, num_v_heads, head_k_dim, head_v_dim, conv_kernel=4,
               l2_eps=1e-6, rms_eps=1e-6, act_dtype="bf16", out_dtype="f32") -> GdnShape:
    code = {"f32": GDN_F32, "bf16": GDN_BF16, GDN_F32: GDN_F32, GDN_BF16: GDN_BF16}
    return GdnShape(int(batch), int(num_k_heads), int(num_v_heads), int(head_k_dim), int(head_v_dim),
                    int(conv_kernel), float(l2_eps), float(rms_eps),
                    code.get(act_dtype, act_dtype), code.get(out_dtype, out_dtype))


_lib = None


def library():
    """The loaded libgdn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError("libgdn.so is not built (%s); run "
                               "`python -m gated_deltanet_linear_causal_amd.build`" % path)
        lib = ctypes.CDLL(path)
        P, S, I32 = ctypes.c_void_p, ctypes.POINTER(GdnShape), ctypes.c_int32
        lib.gdn_conv_update.argtypes = [S, P, P, P, P, P]
        lib.gdn_recurrent_step.argtypes = [S, P, P, P, P, P, P, P, P]
        lib.gdn_decode_layer.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.gdn_sequence.argtypes = [S, I32] + [P] * 12 + [ctypes.c_size_t, P]
        lib.gdn_decode_layer_pooled.argtypes = [S, I32] + [P] * 13
        lib.gdn_decode_layer_debug.argtypes = [S] + [P] * 17
        lib.gdn_decode_verify.argtypes = [S, I32] + [P] * 12 + [ctypes.c_size_t, P]
        lib.gdn_decode_commit.argtypes = [S, I32] + [P] * 5 + [ctypes.c_size_t, P]
        lib.gdn_in_proj.argtypes = [S, I32] + [P] * 10
        lib.gdn_out_proj.argtypes = [S, I32] + [P] * 4
        for f in (lib.gdn_conv_update, lib.gdn_recurrent_step, lib.gdn_decode_layer, lib.gdn_sequence,
                  lib.gdn_decode_layer_pooled, lib.gdn_decode_layer_debug, lib.gdn_decode_verify, lib.gdn_decode_commit, lib.gdn_in_proj,
                  lib.gdn_out_proj):
            f.restype = I32
        for f in (lib.gdn_sequence_workspace_bytes, lib.gdn_verify_trail_bytes):
            f.argtypes = [S, I32]
            f.restype = ctypes.c_size_t
        lib.gdn_status_string.argtypes = [I32]
        lib.gdn_status_string.restype = ctypes.c_char_p
        lib.gdn_abi_version.argtypes = []
        lib.gdn_abi_version.restype = I32
        _lib = lib
    return _lib


def gdn_status_string(status: int) -> str:
    return library().gdn_status_string(int(status)).decode()


def gdn_abi_version() -> int:
    return library().gdn_abi_version()


def gdn_sequence_workspace_bytes(shape: GdnShape, T: int) -> int:
    return library().gdn_sequence_workspace_bytes(ctypes.byref(shape), int(T))


def gdn_verify_trail_bytes(shape: GdnShape, T: int) -> int:
    return library().gdn_verify_trail_bytes(ctypes.byref(shape), int(T))


_ACT = {GDN_F32: torch.float32, GDN_BF16: torch.bfloat16}


def _p(t: Optional[torch.Tensor], name: str, dtype=None, numel: Optional[int] = None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s has %d elements, the shape needs %d" % (name, t.numel(), numel))
    return t.data_ptr()  # an int: the c_void_p argtypes convert it


def _ptr(t: Optional[torch.Tensor], name: str = "", dtype=None, numel: Optional[int] = None):
    """The pointer alone, for validate=False: a caller that has checked its buffers once
    (device, contiguity, dtype, size) skips the per-call checks; the library still checks
    null pointers, alignment, aliasing and the shape."""
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _done(st: int, where: str, check: bool) -> int:
    if check and st != 0:
        raise GdnError(st, where)
    return st


def gdn_conv_update(shape: GdnShape, conv1d_state, qkv, conv1d_weight, qkv_act, stream=None, check=True,
                    validate=True) -> int:
    P = _p if validate else _ptr
    s = shape
    act = _ACT.get(s.act_dtype)
    B, C, K = s.batch, s.channels, s.conv_kernel
    st = library().gdn_conv_update(
        ctypes.byref(s), P(conv1d_state, "conv1d_state", act, B * (K - 1) * C), P(qkv, "qkv", act, B * C),
        P(conv1d_weight, "conv1d_weight", act, C * K), P(qkv_act, "qkv_act", torch.float32, B * C), _stream(stream))
    return _done(st, "gdn_conv_update", check)


def gdn_recurrent_step(shape: GdnShape, state, qkv_act, dt_raw, b_raw, A_log, dt_bias, y, stream=None,
                       check=True, validate=True) -> int:
    P = _p if validate else _ptr
    s = shape
    act, out = _ACT.get(s.act_dtype), _ACT.get(s.out_dtype)
    B, C, Hv, dk, dv = s.batch, s.channels, s.num_v_heads, s.head_k_dim, s.head_v_dim
    st = library().gdn_recurrent_step(
        ctypes.byref(s), P(state, "state", torch.float32, B * Hv * dk * dv),
        P(qkv_act, "qkv_act", torch.float32, B * C), P(dt_raw, "dt_raw", act, B * Hv),
        P(b_raw, "b_raw", act, B * Hv), P(A_log, "A_log", torch.float32, Hv),
        P(dt_bias, "dt_bias", torch.float32, Hv), P(y, "y", out, B * Hv * dv), _stream(stream))
    return _done(st, "gdn_recurrent_step", check)


def gdn_decode_layer(shape: GdnShape, conv1d_state, state, qkv, conv1d_weight, dt_raw, b_raw, z, A_log,
                     dt_bias, norm_weight, out, stream=None, check=True, validate=True) -> int:
    P = _p if validate else _ptr
    s = shape
    act, od = _ACT.get(s.act_dtype), _ACT.get(s.out_dtype)
    B, C, K, Hv, dk, dv = s.batch, s.channels, s.conv_kernel, s.num_v_heads, s.head_k_dim, s.head_v_dim
    st = library().gdn_decode_layer(
        ctypes.byref(s), P(conv1d_state, "conv1d_state", act, B * (K - 1) * C),
        P(state, "state", torch.float32, B * Hv * dk * dv), P(qkv, "qkv", act, B * C),
        P(conv1d_weight, "conv1d_weight", act, C * K), P(dt_raw, "dt_raw", act, B * Hv),
        P(b_raw, "b_raw", act, B * Hv), P(z, "z", act, B * Hv * dv), P(A_log, "A_log", torch.float32, Hv),
        P(dt_bias, "dt_bias", torch.float32, Hv), P(norm_weight, "norm_weight", torch.float32, dv),
        P(out, "out", od, B * Hv * dv), _stream(stream))
    return _done(st, "gdn_decode_layer", check)


def gdn_decode_layer_debug(shape: GdnShape, conv1d_state, state, qkv, conv1d_weight, dt_raw, b_raw, z, A_log,
                           dt_bias, norm_weight, out, qkv_act=None, alpha=None, beta=None, y=None, y_norm=None,
                           stream=None, check=True, validate=True) -> int:
    """gdn_decode_layer plus optional fp32 taps (each None or a GPU tensor): qkv_act
    [B][C], alpha and beta [B][H_v], y and y_norm [B][H_v*d_v]."""
    P = _p if validate else _ptr
    s = shape
    act, od = _ACT.get(s.act_dtype), _ACT.get(s.out_dtype)
    B, C, K, Hv, dk, dv = s.batch, s.channels, s.conv_kernel, s.num_v_heads, s.head_k_dim, s.head_v_dim
    f32 = torch.float32
    st = library().gdn_decode_layer_debug(
        ctypes.byref(s), P(conv1d_state, "conv1d_state", act, B * (K - 1) * C),
        P(state, "state", f32, B * Hv * dk * dv), P(qkv, "qkv", act, B * C),
        P(conv1d_weight, "conv1d_weight", act, C * K), P(dt_raw, "dt_raw", act, B * Hv),
        P(b_raw, "b_raw", act, B * Hv), P(z, "z", act, B * Hv * dv), P(A_log, "A_log", f32, Hv),
        P(dt_bias, "dt_bias", f32, Hv), P(norm_weight, "norm_weight", f32, dv),
        P(out, "out", od, B * Hv * dv), P(qkv_act, "qkv_act", f32, B * C), P(alpha, "alpha", f32, B * Hv),
        P(beta, "beta", f32, B * Hv), P(y, "y", f32, B * Hv * dv), P(y_norm, "y_norm", f32, B * Hv * dv),
        _stream(stream))
    return _done(st, "gdn_decode_layer_debug", check)


def gdn_decode_layer_pooled(shape: GdnShape, slots, conv1d_state_pool, state_pool, qkv, conv1d_weight, dt_raw,
                            b_raw, z, A_log, dt_bias, norm_weight, out, stream=None, check=True,
                            validate=True) -> int:
    """gdn_decode_layer with the states in a pool: sequence b uses slot slots[b]
    (int32 GPU tensor [B]; a slot outside the pool skips the sequence). The pool size
    is taken from state_pool's first dimension."""
    P = _p if validate else _ptr
    s = shape
    act, od = _ACT.get(s.act_dtype), _ACT.get(s.out_dtype)
    B, C, K, Hv, dk, dv = s.batch, s.channels, s.conv_kernel, s.num_v_heads, s.head_k_dim, s.head_v_dim
    pool = int(state_pool.shape[0]) if isinstance(state_pool, torch.Tensor) else 0
    st = library().gdn_decode_layer_pooled(
        ctypes.byref(s), pool, P(slots, "slots", torch.int32, B),
        P(conv1d_state_pool, "conv1d_state_pool", act, pool * (K - 1) * C),
        P(state_pool, "state_pool", torch.float32, pool * Hv * dk * dv), P(qkv, "qkv", act, B * C),
        P(conv1d_weight, "conv1d_weight", act, C * K), P(dt_raw, "dt_raw", act, B * Hv),
        P(b_raw, "b_raw", act, B * Hv), P(z, "z", act, B * Hv * dv), P(A_log, "A_log", torch.float32, Hv),
        P(dt_bias, "dt_bias", torch.float32, Hv), P(norm_weight, "norm_weight", torch.float32, dv),
        P(out, "out", od, B * Hv * dv), _stream(stream))
    return _done(st, "gdn_decode_layer_pooled", check)


def gdn_sequence(shape: GdnShape, T: int, conv1d_state, state, qkv, conv1d_weight, dt_raw, b_raw, z, A_log,
                 dt_bias, norm_weight, out, workspace=None, stream=None, check=True, validate=True) -> int:
    P = _p if validate else _ptr
    s = shape
    act, od = _ACT.get(s.act_dtype), _ACT.get(s.out_dtype)
    B, C, K, Hv, dk, dv = s.batch, s.channels, s.conv_kernel, s.num_v_heads, s.head_k_dim, s.head_v_dim
    T = int(T)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().gdn_sequence(
        ctypes.byref(s), T, P(conv1d_state, "conv1d_state", act, B * (K - 1) * C),
        P(state, "state", torch.float32, B * Hv * dk * dv), P(qkv, "qkv", act, B * T * C),
        P(conv1d_weight, "conv1d_weight", act, C * K), P(dt_raw, "dt_raw", act, B * T * Hv),
        P(b_raw, "b_raw", act, B * T * Hv), P(z, "z", act, B * T * Hv * dv),
        P(A_log, "A_log", torch.float32, Hv), P(dt_bias, "dt_bias", torch.float32, Hv),
        P(norm_weight, "norm_weight", torch.float32, dv), P(out, "out", od, B * T * Hv * dv),
        P(workspace, "workspace"), ctypes.c_size_t(ws_bytes), _stream(stream))
    return _done(st, "gdn_sequence", check)


def gdn_decode_verify(shape: GdnShape, T: int, conv1d_state, state, qkv, conv1d_weight, dt_raw, b_raw, z, A_log,
                      dt_bias, norm_weight, out, trail, stream=None, check=True, validate=True) -> int:
    """Outputs of T draft tokens from the current states, which are only read; the
    per-token updates go to `trail` (a GPU tensor of gdn_verify_trail_bytes bytes)."""
    P = _p if validate else _ptr
    s = shape
    act, od = _ACT.get(s.act_dtype), _ACT.get(s.out_dtype)
    B, C, K, Hv, dk, dv = s.batch, s.channels, s.conv_kernel, s.num_v_heads, s.head_k_dim, s.head_v_dim
    T = int(T)
    tr_bytes = 0 if trail is None else trail.numel() * trail.element_size()
    st = library().gdn_decode_verify(
        ctypes.byref(s), T, P(conv1d_state, "conv1d_state", act, B * (K - 1) * C),
        P(state, "state", torch.float32, B * Hv * dk * dv), P(qkv, "qkv", act, B * T * C),
        P(conv1d_weight, "conv1d_weight", act, C * K), P(dt_raw, "dt_raw", act, B * T * Hv),
        P(b_raw, "b_raw", act, B * T * Hv), P(z, "z", act, B * T * Hv * dv),
        P(A_log, "A_log", torch.float32, Hv), P(dt_bias, "dt_bias", torch.float32, Hv),
        P(norm_weight, "norm_weight", torch.float32, dv), P(out, "out", od, B * T * Hv * dv),
        P(trail, "trail"), ctypes.c_size_t(tr_bytes), _stream(stream))
    return _done(st, "gdn_decode_verify", check)


def gdn_decode_commit(shape: GdnShape, T: int, accepted, conv1d_state, state, qkv, trail, stream=None,
                      check=True, validate=True) -> int:
    """Advance sequence b by its first accepted[b] draft tokens (int32 GPU tensor [B])
    of the preceding gdn_decode_verify call with the same T, qkv and trail."""
    P = _p if validate else _ptr
    s = shape
    act = _ACT.get(s.act_dtype)
    B, C, K, Hv, dk, dv = s.batch, s.channels, s.conv_kernel, s.num_v_heads, s.head_k_dim, s.head_v_dim
    T = int(T)
    tr_bytes = 0 if trail is None else trail.numel() * trail.element_size()
    st = library().gdn_decode_commit(
        ctypes.byref(s), T, P(accepted, "accepted", torch.int32, B),
        P(conv1d_state, "conv1d_state", act, B * (K - 1) * C), P(state, "state", torch.float32, B * Hv * dk * dv),
        P(qkv, "qkv", act, B * T * C), P(trail, "trail"), ctypes.c_size_t(tr_bytes), _stream(stream))
    return _done(st, "gdn_decode_commit", check)


def gdn_in_proj(shape: GdnShape, hidden: int, x_norm, w_qkv, w_z, w_a, w_b, qkv, z, dt_raw, b_raw, stream=None,
                check=True, validate=True) -> int:
    """x_norm [B, hidden] -> qkv, z, dt_raw, b_raw (bf16), weights [outputs, hidden] bf16."""
    P = _p if validate else _ptr
    s = shape
    bf = torch.bfloat16
    B, C, Hv, dv, H = s.batch, s.channels, s.num_v_heads, s.head_v_dim, int(hidden)
    st = library().gdn_in_proj(
        ctypes.byref(s), H, P(x_norm, "x_norm", bf, B * H), P(w_qkv, "w_qkv", bf, C * H),
        P(w_z, "w_z", bf, Hv * dv * H), P(w_a, "w_a", bf, Hv * H), P(w_b, "w_b", bf, Hv * H),
        P(qkv, "qkv", bf, B * C), P(z, "z", bf, B * Hv * dv), P(dt_raw, "dt_raw", bf, B * Hv),
        P(b_raw, "b_raw", bf, B * Hv), _stream(stream))
    return _done(st, "gdn_in_proj", check)


def gdn_out_proj(shape: GdnShape, hidden: int, gated, w_out, y, stream=None, check=True,
                 validate=True) -> int:
    """gated [B, H_v*d_v] bf16 -> y [B, hidden] (out dtype), w_out [hidden, H_v*d_v] bf16."""
    P = _p if validate else _ptr
    s = shape
    bf = torch.bfloat16
    od = _ACT.get(s.out_dtype)
    B, Hv, dv, H = s.batch, s.num_v_heads, s.head_v_dim, int(hidden)
    st = library().gdn_out_proj(
        ctypes.byref(s), H, P(gated, "gated", bf, B * Hv * dv), P(w_out, "w_out", bf, H * Hv * dv),
        P(y, "y", od, B * H), _stream(stream))
    return _done(st, "gdn_out_proj", check)
