"""Shared helpers of the GPU parity tests: seeded inputs to device tensors, runs of
the HIP path through the C-ABI binding, runs of the fp64 oracle on the same inputs,
and the comparison rule.

Tolerance rule (the stricter reading of "max-abs A and max-rel R"): the largest
absolute difference must be <= A, and the largest relative difference over elements
whose reference magnitude is at least REL_FLOOR must be <= R. The conv state is
compared bit for bit.
"""

from __future__ import annotations

import numpy as np
import torch

from gated_deltanet_linear_causal_amd import gdn
from gated_deltanet_linear_causal_amd import inputs as I
from oracle import oracle as O

# (atol, rtol, rel_floor) per activation dtype
TOL = {"bf16": (2e-3, 1e-2, 1e-3), "f32": (1e-5, 1e-5, 1e-1)}


def dev(a: np.ndarray, act: str) -> torch.Tensor:
    """numpy array in storage dtype -> contiguous GPU tensor (bf16 bits or float32)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """GPU tensor -> numpy raw storage (uint16 bits for bf16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    return t.numpy().astype(np.float64)


def shape_for(cfg, batch=None, out_dtype="f32") -> gdn.GdnShape:
    return gdn.make_shape(cfg.batch if batch is None else batch, cfg.num_k_heads, cfg.num_v_heads,
                          cfg.head_k_dim, cfg.head_v_dim, cfg.conv_kernel, cfg.l2_eps, cfg.rms_eps,
                          cfg.act_dtype, out_dtype)


class DeviceInputs:
    """All inputs of a config resident on the GPU (states are fresh copies)."""

    def __init__(self, cfg, data):
        ad = cfg.act_dtype
        self.cfg = cfg
        self.conv_w = dev(data["conv_w"], ad)
        self.A_log = dev(data["A_log"], "f32")
        self.dt_bias = dev(data["dt_bias"], "f32")
        self.norm_w = dev(data["norm_w"], "f32")
        self.state = dev(data["state"], "f32")
        self.conv_state = dev(data["conv_state"], ad)
        self.qkv = dev(data["qkv"], ad)
        self.z = dev(data["z"], ad)
        self.a = dev(data["a"], ad)
        self.b = dev(data["b"], ad)


def gpu_decode(cfg, d: DeviceInputs, steps: int, out_dtype="f32"):
    """`steps` fused decode steps; returns outputs [S, B, H_v*d_v] (torch, on GPU)."""
    s = shape_for(cfg, out_dtype=out_dtype)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    outs = torch.empty((steps, cfg.batch, cfg.z_dim), dtype=od, device="cuda")
    for t in range(steps):
        gdn.gdn_decode_layer(s, d.conv_state, d.state, d.qkv[t], d.conv_w, d.a[t], d.b[t], d.z[t], d.A_log,
                             d.dt_bias, d.norm_w, outs[t])
    torch.cuda.synchronize()
    return outs


def oracle_decode(cfg, data, steps: int, seqs=None):
    """Oracle over `steps` decode steps for the sequences `seqs` (all if None).
    Returns (out [S, nb, H_v*d_v], final state, final conv state), float64."""
    ad = cfg.act_dtype
    idx = np.arange(cfg.batch) if seqs is None else np.asarray(seqs)
    s = O.shape_of(cfg, batch=len(idx))
    cs = I.widen(data["conv_state"][idx], ad).astype(np.float64)
    st = data["state"][idx].astype(np.float64)
    wt = I.widen(data["conv_w"], ad)
    # [S, B, ...] -> [nb, S, ...] so the oracle runs the steps as one sequence call
    sl = lambda k: np.ascontiguousarray(np.swapaxes(I.widen(data[k][:steps][:, idx], ad), 0, 1))
    out = O.sequence(s, steps, cs, st, sl("qkv"), wt, sl("a"), sl("b"), sl("z"), data["A_log"],
                     data["dt_bias"], data["norm_w"])
    return np.swapaxes(out, 0, 1), st, cs


def oracle_sequence(cfg, data, seqs=None):
    ad = cfg.act_dtype
    idx = np.arange(cfg.batch) if seqs is None else np.asarray(seqs)
    s = O.shape_of(cfg, batch=len(idx))
    cs = I.widen(data["conv_state"][idx], ad).astype(np.float64)
    st = data["state"][idx].astype(np.float64)
    w = lambda k: np.ascontiguousarray(I.widen(data[k][idx], ad))
    out = O.sequence(s, cfg.steps, cs, st, w("qkv"), I.widen(data["conv_w"], ad), w("a"), w("b"), w("z"),
                     data["A_log"], data["dt_bias"], data["norm_w"])
    return out, st, cs


def conv_state_bits_expected(cs64: np.ndarray, act: str) -> np.ndarray:
    """The oracle's conv state holds storage values exactly; return them as raw bits."""
    if act == "bf16":
        f = cs64.astype(np.float32)
        assert np.array_equal(f.astype(np.float64), cs64)
        bits = I.f32_to_bf16_bits(f)
        assert np.array_equal(I.bf16_bits_to_f32(bits).astype(np.float64), cs64)
        return bits
    f = cs64.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), cs64)
    return f


def compare(name, got, ref, act, tol=None):
    """Assert the tolerance rule; returns (max_abs, max_rel)."""
    atol, rtol, floor = TOL[act] if tol is None else tol
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % name
    diff = np.abs(got - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    big = np.abs(ref) >= floor
    max_rel = float((diff[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    print("%-40s max_abs %.3e  max_rel %.3e  (atol %.0e rtol %.0e)" % (name, max_abs, max_rel, atol, rtol))
    assert max_abs <= atol, "%s: max abs diff %.3e > %.1e" % (name, max_abs, atol)
    assert max_rel <= rtol, "%s: max rel diff %.3e > %.1e" % (name, max_rel, rtol)
    return max_abs, max_rel


def extreme_inputs(data, seq_major, rng):
    """Gate inputs at the ends of their range: b = -30 / 0 / 30 gives beta ~ 1e-13, 1/2
    and 1; dt = -30 / -8 / 0 / 8 / 30 with A_log up to ln 16 gives log alpha from
    ~-1e-12 (alpha = 1 in fp32) to -480 (alpha = 0 in fp32), so the running log-gate sum
    of a 32-token chunk reaches ~-15000. z takes -20 / -2 / 0.5 / 3, and sequence 0 has
    a zero conv state and all-zero activations at every token: its conv outputs are 0, the
    L2 and RMS norms divide 0 by their epsilon root, its recurrent state only decays, and
    its outputs are exactly 0. Sequence 1 has activations 64 times larger than drawn."""
    bf = lambda x: I.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    data["a"] = bf(rng.choice([-30.0, -8.0, 0.0, 8.0, 30.0], size=data["a"].shape))
    data["b"] = bf(rng.choice([-30.0, 0.0, 30.0], size=data["b"].shape))
    data["z"] = bf(rng.choice([-20.0, -2.0, 0.5, 3.0], size=data["z"].shape))
    data["conv_state"][0] = 0
    # sequence 1: activations 64 times larger (exact in bf16), so v, delta and the
    # state grow by that factor while q and k are normalised
    big = lambda x: I.f32_to_bf16_bits(I.bf16_bits_to_f32(x) * np.float32(64.0))
    if seq_major:
        data["qkv"][0] = 0
        data["qkv"][1] = big(data["qkv"][1])
    else:
        data["qkv"][:, 0] = 0
        data["qkv"][:, 1] = big(data["qkv"][:, 1])
    return data
