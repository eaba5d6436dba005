"""Seeded synthetic inputs for the GDN decode path.

This module is shared by the HIP path's tests/bench and by the fp64 oracle's
callers. It holds only random draws, storage-dtype conversion (fp32 -> bf16 by
round-to-nearest-even) and shape bookkeeping: none of the layer's arithmetic.

Shapes follow the Qwen3.5-style GDN layer on the page "linear_attention.rs"
(spark_model/forward/qwen3_5): qkv is Q | K | V (step 6), one gate and one beta per
v-head (steps 4-5), a per-head state (step 7), per-head norm weight of d_v
(step 8). The conv state is [K-1, C] per sequence, time-major, rolled in place
(page "ple.rs", doc of ple_conv).

Recipe (all draws from ``numpy.random.default_rng(seed)`` in this order):
  1. parameters: conv_w [C, K] ~ N(0, 0.5); A_log [H_v] ~ U(0, ln 16);
     dt_bias [H_v] = softplus^-1(u), u ~ U(1e-3, 0.1); norm_w [d_v] = 1 + N(0, 0.1)
  2. initial states: recurrent state [B, H_v, d_k, d_v] ~ N(0, state_std) (or 0),
     then conv state [B, K-1, C] ~ N(0, conv_state_std) (or 0)
  3. per decode step (in step order): qkv [B, C], z [B, H_v*d_v], a [B, H_v],
     b [B, H_v], all N(0, 1); for a sequence the same four arrays are drawn
     once each with a T axis after B.
Normal draws are made in float32 (``standard_normal(dtype=float32)``) and scaled;
where the activation dtype is bf16 they are rounded RNE to bf16. Recurrent state
and A_log, dt_bias, norm_w stay fp32.

Projections around the layer (``generate_projections``, own seed): x_norm [B, hidden]
~ N(0, 1), then w_qkv [C, hidden], w_z [H_v*d_v, hidden], w_a [H_v, hidden], w_b
[H_v, hidden] ~ N(0, 1/hidden) and w_out [hidden, H_v*d_v] ~ N(0, 1/(H_v*d_v)), all
rounded to bf16. The pages do not give the model's hidden size; HIDDEN is the value
used for measurements.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "GdnConfig",
    "CONFIGS",
    "config",
    "generate",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "widen",
]


@dataclasses.dataclass(frozen=True)
class GdnConfig:
    name: str
    batch: int
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int
    head_v_dim: int
    conv_kernel: int
    act_dtype: str  # "f32" or "bf16": qkv, z, a, b, conv_w, conv state
    steps: int  # decode steps, or T for a sequence
    seed: int
    mode: str = "decode"  # "decode" (steps separate calls) or "sequence" (one call)
    state_std: float = 0.0  # 0 -> zero initial recurrent state
    conv_state_std: float = 0.0  # 0 -> zero initial conv state
    l2_eps: float = 1e-6
    rms_eps: float = 1e-6

    @property
    def channels(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    @property
    def z_dim(self) -> int:
        return self.num_v_heads * self.head_v_dim

    @property
    def group(self) -> int:
        return self.num_v_heads // self.num_k_heads

    def with_(self, **kw) -> "GdnConfig":
        return dataclasses.replace(self, **kw)


def _qwen35(name, batch, steps, seed, mode="decode", state_std=0.02, conv_state_std=1.0):
    return GdnConfig(
        name=name, batch=batch, num_k_heads=16, num_v_heads=32, head_k_dim=128,
        head_v_dim=128, conv_kernel=4, act_dtype="bf16", steps=steps, seed=seed,
        mode=mode, state_std=state_std, conv_state_std=conv_state_std)


# The five workloads. Index = seed for the Qwen3.5-style ones.
CONFIGS = [
    GdnConfig(name="tiny_fp32_B1", batch=1, num_k_heads=2, num_v_heads=2, head_k_dim=32,
              head_v_dim=32, conv_kernel=4, act_dtype="f32", steps=16, seed=0),
    _qwen35("qwen35_B1", batch=1, steps=1, seed=1),
    _qwen35("qwen35_B64", batch=64, steps=32, seed=2),
    _qwen35("qwen35_B512", batch=512, steps=32, seed=3),
    _qwen35("qwen35_seq_B8_T4096", batch=8, steps=4096, seed=4, mode="sequence",
            state_std=0.0, conv_state_std=0.0),
]


def config(i: int) -> GdnConfig:
    return CONFIGS[i]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(a: np.ndarray, act_dtype: str) -> np.ndarray:
    """Exact float32 view of an activation-dtype array (bf16 bits or float32)."""
    if act_dtype == "bf16":
        return bf16_bits_to_f32(a)
    return np.ascontiguousarray(a, dtype=np.float32)


def _act(x32: np.ndarray, act_dtype: str) -> np.ndarray:
    if act_dtype == "bf16":
        return f32_to_bf16_bits(x32)
    return np.ascontiguousarray(x32, dtype=np.float32)


def _normal(rng, shape, std):
    out = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def generate(cfg: GdnConfig, steps: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every input of ``cfg``.

    Returns a dict with: ``conv_w`` [C, K] (act dtype), ``A_log``, ``dt_bias`` [H_v]
    and ``norm_w`` [d_v] (float32), ``state`` [B, H_v, d_k, d_v] (float32),
    ``conv_state`` [B, K-1, C] (act dtype); then for decode mode ``qkv`` [S, B, C],
    ``z`` [S, B, H_v*d_v], ``a`` [S, B, H_v], ``b`` [S, B, H_v] with S steps, and for
    sequence mode the same names shaped [B, T, ...]. Act-dtype arrays are uint16
    bf16 bits or float32.
    """
    steps = cfg.steps if steps is None else steps
    rng = np.random.default_rng(cfg.seed)
    B, Hv, dk, dv, K, C = (cfg.batch, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim,
                           cfg.conv_kernel, cfg.channels)
    ad = cfg.act_dtype
    out: Dict[str, np.ndarray] = {}
    # 1. parameters
    out["conv_w"] = _act(_normal(rng, (C, K), 0.5), ad)
    out["A_log"] = rng.uniform(0.0, math.log(16.0), size=Hv).astype(np.float32)
    u = rng.uniform(1e-3, 0.1, size=Hv)
    out["dt_bias"] = np.log(np.expm1(u)).astype(np.float32)  # softplus^-1(u)
    out["norm_w"] = (1.0 + _normal(rng, (dv,), 0.1)).astype(np.float32)
    # 2. initial states
    if cfg.state_std > 0:
        out["state"] = _normal(rng, (B, Hv, dk, dv), cfg.state_std)
    else:
        out["state"] = np.zeros((B, Hv, dk, dv), dtype=np.float32)
    if cfg.conv_state_std > 0:
        out["conv_state"] = _act(_normal(rng, (B, K - 1, C), cfg.conv_state_std), ad)
    else:
        out["conv_state"] = _act(np.zeros((B, K - 1, C), dtype=np.float32), ad)
    # 3. per-step activations
    if cfg.mode == "sequence":
        T = steps
        out["qkv"] = _act(_normal(rng, (B, T, C), 1.0), ad)
        out["z"] = _act(_normal(rng, (B, T, Hv * dv), 1.0), ad)
        out["a"] = _act(_normal(rng, (B, T, Hv), 1.0), ad)
        out["b"] = _act(_normal(rng, (B, T, Hv), 1.0), ad)
    else:
        q = np.empty((steps, B, C), dtype=np.uint16 if ad == "bf16" else np.float32)
        z = np.empty((steps, B, Hv * dv), dtype=q.dtype)
        a = np.empty((steps, B, Hv), dtype=q.dtype)
        b = np.empty((steps, B, Hv), dtype=q.dtype)
        for s in range(steps):
            q[s] = _act(_normal(rng, (B, C), 1.0), ad)
            z[s] = _act(_normal(rng, (B, Hv * dv), 1.0), ad)
            a[s] = _act(_normal(rng, (B, Hv), 1.0), ad)
            b[s] = _act(_normal(rng, (B, Hv), 1.0), ad)
        out["qkv"], out["z"], out["a"], out["b"] = q, z, a, b
    return out


HIDDEN = 2048


def generate_projections(cfg: GdnConfig, hidden: int = HIDDEN, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Synthetic input and weights of the in_proj / out_proj steps (bf16 bits, uint16):
    ``x_norm`` [B, hidden], ``w_qkv`` [C, hidden], ``w_z`` [H_v*d_v, hidden], ``w_a`` and
    ``w_b`` [H_v, hidden], ``w_out`` [hidden, H_v*d_v]. Weights are scaled by
    1/sqrt(fan_in) so the outputs are O(1)."""
    rng = np.random.default_rng(cfg.seed + 7919 if seed is None else seed)
    B, Hv, dv, C = cfg.batch, cfg.num_v_heads, cfg.head_v_dim, cfg.channels
    zd = Hv * dv
    out: Dict[str, np.ndarray] = {}
    out["x_norm"] = _act(_normal(rng, (B, hidden), 1.0), "bf16")
    s_in = 1.0 / math.sqrt(hidden)
    out["w_qkv"] = _act(_normal(rng, (C, hidden), s_in), "bf16")
    out["w_z"] = _act(_normal(rng, (zd, hidden), s_in), "bf16")
    out["w_a"] = _act(_normal(rng, (Hv, hidden), s_in), "bf16")
    out["w_b"] = _act(_normal(rng, (Hv, hidden), s_in), "bf16")
    out["w_out"] = _act(_normal(rng, (hidden, zd), 1.0 / math.sqrt(zd)), "bf16")
    return out
