"""Python access to the fp64 CPU oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline leg use this module. It marshals numpy arrays into the C oracle and
widens every input exactly (float32 or bf16 values -> the C code's double
arithmetic); it does no arithmetic of the layer itself.

The C library is compiled with gcc (``-O2 -fopenmp -ffp-contract=off``, no fast-math)
into ``oracle/_build/libgdn_oracle.so`` on first use, or by :func:`build`.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_HDR = os.path.join(_HERE, "gdn_oracle.h")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libgdn_oracle.so")


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-I", _HERE, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int), ("num_k_heads", ctypes.c_int),
                ("num_v_heads", ctypes.c_int), ("head_k_dim", ctypes.c_int),
                ("head_v_dim", ctypes.c_int), ("conv_kernel", ctypes.c_int),
                ("l2_eps", ctypes.c_double), ("rms_eps", ctypes.c_double)]


_lib = None


def _load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))):
            build(force=True)
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


class use_library:
    """Context manager that points this module at another build of the oracle
    (used by the test that plants mistakes in copies of the oracle source)."""

    def __init__(self, path: str):
        self.path = path
        self.saved = None

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _bind(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _bind(lib):
    P = ctypes.c_void_p
    S = ctypes.POINTER(_Shape)
    lib.gdn_oracle_check_shape.argtypes = [S]
    lib.gdn_oracle_check_shape.restype = ctypes.c_int
    lib.gdn_oracle_threads.argtypes = [ctypes.c_int]
    lib.gdn_oracle_threads.restype = ctypes.c_int
    lib.gdn_oracle_conv_update.argtypes = [S, P, P, P, P]
    lib.gdn_oracle_recurrent_step.argtypes = [S, P, P, P, P, P, P, P, P, P]
    lib.gdn_oracle_gated_rmsnorm.argtypes = [S, P, P, P, P, P]
    lib.gdn_oracle_decode_step.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P]
    lib.gdn_oracle_sequence.argtypes = [S, ctypes.c_int] + [P] * 11
    lib.gdn_oracle_linear.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P]
    for f in (lib.gdn_oracle_conv_update, lib.gdn_oracle_recurrent_step, lib.gdn_oracle_gated_rmsnorm,
              lib.gdn_oracle_decode_step, lib.gdn_oracle_sequence, lib.gdn_oracle_linear):
        f.restype = None
    return lib


def shape_of(cfg, batch: Optional[int] = None, l2_eps: Optional[float] = None,
             rms_eps: Optional[float] = None) -> _Shape:
    """Oracle shape from any object with the GdnConfig attribute names."""
    s = _Shape(batch=cfg.batch if batch is None else batch, num_k_heads=cfg.num_k_heads,
               num_v_heads=cfg.num_v_heads, head_k_dim=cfg.head_k_dim,
               head_v_dim=cfg.head_v_dim, conv_kernel=cfg.conv_kernel,
               l2_eps=cfg.l2_eps if l2_eps is None else l2_eps,
               rms_eps=cfg.rms_eps if rms_eps is None else rms_eps)
    rc = _load().gdn_oracle_check_shape(ctypes.byref(s))
    if rc != 0:
        raise ValueError("invalid GDN shape for the oracle (code %d)" % rc)
    return s


def threads(n: int = 0) -> int:
    """Set (n > 0) and return the oracle's OpenMP thread count."""
    return _load().gdn_oracle_threads(int(n))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dims(s: _Shape):
    C = 2 * s.num_k_heads * s.head_k_dim + s.num_v_heads * s.head_v_dim
    return s.batch, C, s.num_v_heads, s.head_v_dim, s.head_k_dim, s.conv_kernel


def _check(a: np.ndarray, shape, name):
    if tuple(a.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), a.shape))


def conv_update(s: _Shape, conv_state: np.ndarray, qkv, conv_w) -> np.ndarray:
    """Step 3: rolls ``conv_state`` (float64, [B, K-1, C], in place); returns qkv_act."""
    B, C, Hv, dv, dk, K = _dims(s)
    _check(conv_state, (B, K - 1, C), "conv_state")
    assert conv_state.dtype == np.float64 and conv_state.flags.c_contiguous
    qkv, conv_w = _f32(qkv), _f32(conv_w)
    _check(qkv, (B, C), "qkv")
    _check(conv_w, (C, K), "conv_w")
    act = np.zeros((B, C), dtype=np.float64)
    _load().gdn_oracle_conv_update(ctypes.byref(s), _ptr(conv_state), _ptr(qkv), _ptr(conv_w), _ptr(act))
    return act


def recurrent_step(s: _Shape, state: np.ndarray, qkv_act, dt_raw, b_raw, A_log, dt_bias
                   ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Steps 4, 5, 7: updates ``state`` (float64 in place); returns (o, alpha, beta)."""
    B, C, Hv, dv, dk, K = _dims(s)
    _check(state, (B, Hv, dk, dv), "state")
    assert state.dtype == np.float64 and state.flags.c_contiguous
    qkv_act = _f64(qkv_act)
    _check(qkv_act, (B, C), "qkv_act")
    dt_raw, b_raw, A_log, dt_bias = _f32(dt_raw), _f32(b_raw), _f32(A_log), _f32(dt_bias)
    _check(dt_raw, (B, Hv), "dt_raw")
    _check(b_raw, (B, Hv), "b_raw")
    _check(A_log, (Hv,), "A_log")
    _check(dt_bias, (Hv,), "dt_bias")
    o = np.zeros((B, Hv, dv), dtype=np.float64)
    alpha = np.zeros((B, Hv), dtype=np.float64)
    beta = np.zeros((B, Hv), dtype=np.float64)
    _load().gdn_oracle_recurrent_step(ctypes.byref(s), _ptr(state), _ptr(qkv_act), _ptr(dt_raw),
                                      _ptr(b_raw), _ptr(A_log), _ptr(dt_bias), _ptr(o),
                                      _ptr(alpha), _ptr(beta))
    return o, alpha, beta


def gated_rmsnorm(s: _Shape, o, z, norm_w) -> Tuple[np.ndarray, np.ndarray]:
    """Step 8 and the silu(z) gate: returns (y_norm, out), both [B, H_v*d_v]."""
    B, C, Hv, dv, dk, K = _dims(s)
    o = _f64(o).reshape(B, Hv * dv)
    z, norm_w = _f32(z).reshape(B, Hv * dv), _f32(norm_w)
    _check(norm_w, (dv,), "norm_w")
    y_norm = np.zeros((B, Hv * dv), dtype=np.float64)
    out = np.zeros((B, Hv * dv), dtype=np.float64)
    _load().gdn_oracle_gated_rmsnorm(ctypes.byref(s), _ptr(o), _ptr(z), _ptr(norm_w), _ptr(y_norm), _ptr(out))
    return y_norm, out


def decode_step(s: _Shape, conv_state: np.ndarray, state: np.ndarray, qkv, conv_w, dt_raw, b_raw,
                z, A_log, dt_bias, norm_w) -> np.ndarray:
    """One whole decode step; updates both states in place; returns out [B, H_v*d_v]."""
    return sequence(s, 1, conv_state, state, np.asarray(qkv)[:, None], conv_w,
                    np.asarray(dt_raw)[:, None], np.asarray(b_raw)[:, None],
                    np.asarray(z)[:, None], A_log, dt_bias, norm_w)[:, 0]


def sequence(s: _Shape, T: int, conv_state: np.ndarray, state: np.ndarray, qkv, conv_w, dt_raw,
             b_raw, z, A_log, dt_bias, norm_w) -> np.ndarray:
    """T decode steps per sequence (inputs [B, T, ...]); returns out [B, T, H_v*d_v]."""
    B, C, Hv, dv, dk, K = _dims(s)
    _check(conv_state, (B, K - 1, C), "conv_state")
    _check(state, (B, Hv, dk, dv), "state")
    for a, nm in ((conv_state, "conv_state"), (state, "state")):
        if a.dtype != np.float64 or not a.flags.c_contiguous:
            raise ValueError("%s must be a C-contiguous float64 array" % nm)
    qkv, conv_w = _f32(qkv), _f32(conv_w)
    dt_raw, b_raw, z = _f32(dt_raw), _f32(b_raw), _f32(z)
    A_log, dt_bias, norm_w = _f32(A_log), _f32(dt_bias), _f32(norm_w)
    _check(qkv, (B, T, C), "qkv")
    _check(conv_w, (C, K), "conv_w")
    _check(dt_raw, (B, T, Hv), "dt_raw")
    _check(b_raw, (B, T, Hv), "b_raw")
    _check(z, (B, T, Hv * dv), "z")
    _check(A_log, (Hv,), "A_log")
    _check(dt_bias, (Hv,), "dt_bias")
    _check(norm_w, (dv,), "norm_w")
    out = np.zeros((B, T, Hv * dv), dtype=np.float64)
    _load().gdn_oracle_sequence(ctypes.byref(s), int(T), _ptr(conv_state), _ptr(state), _ptr(qkv),
                                _ptr(conv_w), _ptr(dt_raw), _ptr(b_raw), _ptr(z), _ptr(A_log),
                                _ptr(dt_bias), _ptr(norm_w), _ptr(out))
    return out


def linear(x, w) -> np.ndarray:
    """y[m][n] = sum_k x[m][k] w[n][k] in fp64 (x [M, K], w [N, K] exact float values):
    the projections on either side of the layer ("linear_attention.rs", step 2 and
    steps 9-11). Returns y [M, N] float64."""
    x, w = _f32(x), _f32(w)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("linear: x [M, K] and w [N, K] expected, got %s and %s" % (x.shape, w.shape))
    M, K = x.shape
    N = w.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    _load().gdn_oracle_linear(int(M), int(N), int(K), _ptr(x), _ptr(w), _ptr(y))
    return y
