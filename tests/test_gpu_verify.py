"""Speculative decoding through the C-ABI: gdn_decode_verify (T draft tokens, states
read only) and gdn_decode_commit (advance each sequence by its accepted prefix),
against the fp64 oracle run token by token.

* verify's outputs for all T draft tokens == the oracle's T-token sequence from the
  same states (tolerance rule of gdn_cases);
* both states are bit-for-bit unchanged by verify;
* after commit with per-sequence counts n_b (0, 1, T and values in between) the
  state == the oracle's state after n_b tokens, the conv state == the oracle's rolled
  conv state bit for bit, and sequences with n_b = 0 or n_b outside [0, T] are
  untouched;
* verifying the remaining draft tokens from the committed state gives the first
  verify's outputs up to fp32 rounding (the first formed them from the state before
  the draft, the second from the replayed state).
"""

import numpy as np
import pytest
import torch

from gated_deltanet_linear_causal_amd import gdn
from gated_deltanet_linear_causal_amd import inputs as I
from oracle import oracle as O

from gdn_cases import TOL, compare, conv_state_bits_expected, dev, extreme_inputs, host_bits, host_f64, shape_for

pytestmark = pytest.mark.gpu


def tol_of(act, d):
    """bf16 activations: the workload bound. fp32 activations: 1e-5, the bound stated
    for the all-fp32 layer (verify evaluates the unrolled rule and commit replays the
    updates, both in fp32 with no reduced-precision operands)."""
    if act == "bf16":
        return TOL["bf16"]
    return (1e-5, 1e-5, 1e-1)


def cfg_of(name, B, Hk, Hv, d, K, act, T):
    return I.GdnConfig(name=name, batch=B, num_k_heads=Hk, num_v_heads=Hv, head_k_dim=d, head_v_dim=d,
                       conv_kernel=K, act_dtype=act, steps=T, seed=2000 + B * 7 + Hv * 3 + d + K + T,
                       mode="sequence", state_std=0.02, conv_state_std=1.0)


CASES = [
    # name, B, Hk, Hv, d, K, act, T, accepted per sequence
    ("qwen35_B4_T4", 4, 16, 32, 128, 4, "bf16", 4, [0, 1, 4, 2]),
    ("qwen35_B3_T8", 3, 16, 32, 128, 4, "bf16", 8, [8, 5, 3]),
    ("tiny_f32_T8", 2, 2, 2, 32, 4, "f32", 8, [7, 8]),
    ("G4_d64_K3_T6", 3, 2, 8, 64, 3, "bf16", 6, [6, 0, 4]),
    ("G3_d128_K2_T5_f32", 2, 1, 3, 128, 2, "f32", 5, [2, 5]),
    ("G2_d32_K6_T3", 5, 2, 4, 32, 6, "bf16", 3, [1, 3, 0, 2, 3]),
    ("T1_B2", 2, 16, 32, 128, 4, "bf16", 1, [1, 0]),
    # the benchmark's verify workload: B = 64, 4 draft tokens, every count 0..4
    ("qwen35_B64_T4", 64, 16, 32, 128, 4, "bf16", 4, [i % 5 for i in range(64)]),
]


class Case:
    def __init__(self, name, B, Hk, Hv, d, K, act, T, extreme=False):
        self.cfg = cfg_of(name, B, Hk, Hv, d, K, act, T)
        self.data = I.generate(self.cfg)
        if extreme:
            extreme_inputs(self.data, True, np.random.default_rng(T))
        ad = act
        dd = self.data
        self.conv_w = dev(dd["conv_w"], ad)
        self.A_log = dev(dd["A_log"], "f32")
        self.dt_bias = dev(dd["dt_bias"], "f32")
        self.norm_w = dev(dd["norm_w"], "f32")
        self.state = dev(dd["state"], "f32")
        self.conv_state = dev(dd["conv_state"], ad)
        self.qkv = dev(dd["qkv"], ad)
        self.z = dev(dd["z"], ad)
        self.a = dev(dd["a"], ad)
        self.b = dev(dd["b"], ad)
        self.shape = shape_for(self.cfg)
        self.trail = torch.empty(gdn.gdn_verify_trail_bytes(self.shape, T), dtype=torch.uint8, device="cuda")

    def verify(self, T=None, qkv=None, z=None, a=None, b=None):
        c = self.cfg
        T = c.steps if T is None else T
        out = torch.full((c.batch, T, c.z_dim), float("nan"), dtype=torch.float32, device="cuda")
        gdn.gdn_decode_verify(self.shape, T, self.conv_state, self.state, self.qkv if qkv is None else qkv,
                              self.conv_w, self.a if a is None else a, self.b if b is None else b,
                              self.z if z is None else z, self.A_log, self.dt_bias, self.norm_w, out, self.trail)
        torch.cuda.synchronize()
        return out

    def commit(self, accepted, T=None, qkv=None):
        T = self.cfg.steps if T is None else T
        acc = torch.tensor(accepted, dtype=torch.int32, device="cuda")
        gdn.gdn_decode_commit(self.shape, T, acc, self.conv_state, self.state, self.qkv if qkv is None else qkv,
                              self.trail)
        torch.cuda.synchronize()


def oracle_prefix(cfg, data, b, n):
    """Oracle states of sequence b after its first n tokens (float64)."""
    ad = cfg.act_dtype
    s = O.shape_of(cfg, batch=1)
    cs = I.widen(data["conv_state"][b:b + 1], ad).astype(np.float64)
    st = data["state"][b:b + 1].astype(np.float64)
    if n > 0:
        w = lambda k: np.ascontiguousarray(I.widen(data[k][b:b + 1, :n], ad))
        O.sequence(s, n, cs, st, w("qkv"), I.widen(data["conv_w"], ad), w("a"), w("b"), w("z"),
                   data["A_log"], data["dt_bias"], data["norm_w"])
    return st[0], cs[0]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_verify_then_commit(case):
    name, B, Hk, Hv, d, K, act, T, accepted = case
    print("case", name, flush=True)
    _verify_then_commit(Case(name, B, Hk, Hv, d, K, act, T), accepted)


def test_verify_then_commit_extreme_gates():
    """Gates at the ends of their range and a sequence of all-zero activations (the
    inputs of the decode and sequence edge tests), over 8 draft tokens."""
    print("case extreme_B3_T8", flush=True)
    _verify_then_commit(Case("extreme_B3_T8", 3, 2, 4, 128, 4, "bf16", 8, extreme=True), [8, 3, 0])


def _verify_then_commit(c, accepted):
    cfg, data = c.cfg, c.data
    name, act, d, T = cfg.name, cfg.act_dtype, cfg.head_v_dim, cfg.steps
    tol = tol_of(act, d)
    state0, conv0 = host_bits(c.state).copy(), host_bits(c.conv_state).copy()

    out = c.verify()
    # the states are only read
    assert np.array_equal(host_bits(c.state), state0)
    assert np.array_equal(host_bits(c.conv_state), conv0)
    # every draft token's output, as the oracle's T-token sequence gives it
    s = O.shape_of(cfg)
    cs = I.widen(data["conv_state"], act).astype(np.float64)
    st = data["state"].astype(np.float64)
    w = lambda k: np.ascontiguousarray(I.widen(data[k], act))
    ref = O.sequence(s, T, cs, st, w("qkv"), I.widen(data["conv_w"], act), w("a"), w("b"), w("z"),
                     data["A_log"], data["dt_bias"], data["norm_w"])
    compare(name + " verify out", host_f64(out), ref, act, tol)

    c.commit(accepted)
    got_state, got_conv = host_f64(c.state), host_bits(c.conv_state)
    for b, n in enumerate(accepted):
        st_ref, cs_ref = oracle_prefix(cfg, data, b, n)
        if n == 0:
            assert np.array_equal(host_bits(c.state)[b], state0[b])
            assert np.array_equal(got_conv[b], conv0[b])
        compare("%s state b%d n%d" % (name, b, n), got_state[b], st_ref, act, tol)
        assert np.array_equal(got_conv[b], conv_state_bits_expected(cs_ref, act)), (name, b, n)


def test_commit_then_verify_the_rest():
    """Verify T tokens, commit n, verify the remaining T - n from the committed state:
    those outputs equal the first verify's up to fp32 rounding (same bf16 inputs; the
    first verify unrolled the rule from the state before the draft, the second starts
    from the state the commit replayed), for n = 1, 2 and 5 of T = 6."""
    T = 6
    for n in (1, 2, 5):
        c = Case("resume", 3, 16, 32, 128, 4, "bf16", T)
        out_all = c.verify()
        c.commit([n] * c.cfg.batch)
        rest = lambda t: t[:, n:].contiguous()
        c.trail = torch.empty(gdn.gdn_verify_trail_bytes(c.shape, T - n), dtype=torch.uint8, device="cuda")
        out_rest = c.verify(T=T - n, qkv=rest(c.qkv), z=rest(c.z), a=rest(c.a), b=rest(c.b))
        compare("verify after commit of %d" % n, host_f64(out_rest), host_f64(out_all[:, n:]), "f32")


def test_out_of_range_counts_leave_sequences_untouched():
    T = 4
    c = Case("range", 4, 16, 32, 128, 4, "bf16", T)
    state0, conv0 = host_bits(c.state).copy(), host_bits(c.conv_state).copy()
    c.verify()
    c.commit([-1, T + 1, 0, 2 ** 31 - 1])
    assert np.array_equal(host_bits(c.state), state0)
    assert np.array_equal(host_bits(c.conv_state), conv0)


def test_bf16_output():
    """out_dtype bf16: each value is the fp32 result rounded to nearest even (one ulp
    of bf16 from the fp32 run's value)."""
    T = 4
    c = Case("bf16out", 2, 16, 32, 128, 4, "bf16", T)
    ref = c.verify()
    s16 = shape_for(c.cfg, out_dtype="bf16")
    out16 = torch.empty((c.cfg.batch, T, c.cfg.z_dim), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_decode_verify(s16, T, c.conv_state, c.state, c.qkv, c.conv_w, c.a, c.b, c.z, c.A_log, c.dt_bias,
                          c.norm_w, out16, c.trail)
    torch.cuda.synchronize()
    r = host_f64(ref)
    g = host_f64(out16)
    assert np.all(np.abs(g - r) <= 2.0 ** -8 * np.abs(r) + 1e-30)
