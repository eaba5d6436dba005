"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with:
  * library routines composed in a different formulation (np.convolve for the causal
    conv, scipy's expit for SiLU/sigmoid, torch's normalize / rms_norm / softplus /
    silu, and the matrix form S <- alpha S (I - beta k k^T) + beta v k^T of the
    published gated delta rule, where the oracle uses a per-column form);
  * closed forms (softplus(0) = ln 2, alpha = sigmoid(-x) when A_log = 0, ...);
  * exact rational arithmetic (fractions.Fraction) on tiny heads;
  * invariants (unit L2 norms, alpha = beta = 1 recall, state roll, resume,
    permutation equivariance over sequences and k-head groups).
The functions are plain so that the mutation test can run the same pins against
copies of the oracle with planted mistakes and check that each is caught.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F
from scipy.special import expit

from oracle import oracle as O


class Shape:
    """A small GDN shape with d_k != d_v and two v-heads per k-head."""

    def __init__(self, batch=2, num_k_heads=2, num_v_heads=4, head_k_dim=8, head_v_dim=6,
                 conv_kernel=4, l2_eps=1e-6, rms_eps=1e-6):
        self.batch, self.num_k_heads, self.num_v_heads = batch, num_k_heads, num_v_heads
        self.head_k_dim, self.head_v_dim, self.conv_kernel = head_k_dim, head_v_dim, conv_kernel
        self.l2_eps, self.rms_eps = l2_eps, rms_eps

    @property
    def channels(self):
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    @property
    def group(self):
        return self.num_v_heads // self.num_k_heads


def draw(sh: Shape, T: int, seed: int, state_std=0.3, conv_std=1.0):
    """Random float32 inputs for a small shape (test-local, not a workload)."""
    rng = np.random.default_rng(seed)
    B, C, K, Hv, dk, dv = sh.batch, sh.channels, sh.conv_kernel, sh.num_v_heads, sh.head_k_dim, sh.head_v_dim
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(
        conv_w=(0.5 * f(C, K)).astype(np.float32),
        A_log=rng.uniform(0, math.log(16), Hv).astype(np.float32),
        dt_bias=np.log(np.expm1(rng.uniform(1e-3, 0.1, Hv))).astype(np.float32),
        norm_w=(1 + 0.1 * f(dv)).astype(np.float32),
        state=(state_std * f(B, Hv, dk, dv)).astype(np.float32),
        conv_state=(conv_std * f(B, K - 1, C)).astype(np.float32),
        qkv=f(B, T, C), z=f(B, T, Hv * dv), a=f(B, T, Hv), b=f(B, T, Hv))


def run_oracle(sh: Shape, x: dict, T: int):
    s = O.shape_of(sh)
    cs = np.ascontiguousarray(x["conv_state"], dtype=np.float64)
    st = np.ascontiguousarray(x["state"], dtype=np.float64)
    out = O.sequence(s, T, cs, st, x["qkv"], x["conv_w"], x["a"], x["b"], x["z"], x["A_log"],
                     x["dt_bias"], x["norm_w"])
    return out, cs, st


# ---------------------------------------------------------------------------------
# An independent composition of library routines, in matrix form.
# ---------------------------------------------------------------------------------

def library_reference(sh: Shape, x: dict, T: int):
    """The layer step composed from library routines (float64), in matrix form."""
    B, C, K, Hk, Hv, dk, dv = (sh.batch, sh.channels, sh.conv_kernel, sh.num_k_heads,
                               sh.num_v_heads, sh.head_k_dim, sh.head_v_dim)
    G = Hv // Hk
    full = np.concatenate([x["conv_state"].astype(np.float64), x["qkv"].astype(np.float64)], axis=1)
    u = np.empty((B, T, C))
    for b in range(B):
        for c in range(C):
            # true convolution with the reversed taps = tap K-1 on the newest sample
            u[b, :, c] = np.convolve(full[b, :, c], x["conv_w"][c, ::-1].astype(np.float64), mode="valid")
    act = u * expit(u)
    q = torch.from_numpy(act[..., :Hk * dk].reshape(B, T, Hk, dk).copy())
    k = torch.from_numpy(act[..., Hk * dk:2 * Hk * dk].reshape(B, T, Hk, dk).copy())
    v = act[..., 2 * Hk * dk:].reshape(B, T, Hv, dv)
    # eps-free unit norm, then the eps factor sqrt(S / (S + eps)) of x / sqrt(S + eps)
    qn = F.normalize(q, dim=-1, eps=0.0) * torch.sqrt((q * q).sum(-1, keepdim=True) /
                                                       ((q * q).sum(-1, keepdim=True) + sh.l2_eps))
    kn = F.normalize(k, dim=-1, eps=0.0) * torch.sqrt((k * k).sum(-1, keepdim=True) /
                                                       ((k * k).sum(-1, keepdim=True) + sh.l2_eps))
    qn, kn = qn.numpy(), kn.numpy()
    xg = torch.from_numpy(x["a"].astype(np.float64) + x["dt_bias"].astype(np.float64))
    sp = F.softplus(xg, beta=1.0, threshold=1e9).numpy()
    alpha = np.exp(-np.exp(x["A_log"].astype(np.float64)) * sp)  # [B, T, Hv]
    beta = expit(x["b"].astype(np.float64))
    S = np.transpose(x["state"].astype(np.float64), (0, 1, 3, 2)).copy()  # [B, Hv, dv, dk]
    o = np.empty((B, T, Hv, dv))
    eye = np.eye(dk)
    for b in range(B):
        for t in range(T):
            for h in range(Hv):
                kk, qq, vv = kn[b, t, h // G], qn[b, t, h // G], v[b, t, h]
                a_, b_ = alpha[b, t, h], beta[b, t, h]
                S[b, h] = a_ * S[b, h] @ (eye - b_ * np.outer(kk, kk)) + b_ * np.outer(vv, kk)
                o[b, t, h] = S[b, h] @ qq / math.sqrt(dk)
    on = F.rms_norm(torch.from_numpy(o), (dv,), weight=torch.from_numpy(x["norm_w"].astype(np.float64)),
                    eps=sh.rms_eps)
    out = on * F.silu(torch.from_numpy(x["z"].astype(np.float64).reshape(B, T, Hv, dv)))
    conv_final = full[:, -(K - 1):, :]
    return (out.numpy().reshape(B, T, Hv * dv), conv_final,
            np.transpose(S, (0, 1, 3, 2)), act, alpha, beta)


def pin_library_composition():
    """Whole steps (conv, SiLU, L2, gates, delta rule, readout, gated norm) over T
    tokens equal the library composition in matrix form."""
    for sh, T, seed in ((Shape(), 7, 11), (Shape(batch=1, num_k_heads=1, num_v_heads=3, head_k_dim=5,
                                                 head_v_dim=7, conv_kernel=3), 5, 12),
                        (Shape(batch=1, conv_kernel=2, head_k_dim=4, head_v_dim=4), 3, 13)):
        x = draw(sh, T, seed)
        out, cs, st = run_oracle(sh, x, T)
        r_out, r_cs, r_st, *_ = library_reference(sh, x, T)
        np.testing.assert_allclose(out, r_out, rtol=0, atol=1e-11)
        np.testing.assert_array_equal(cs, r_cs)
        np.testing.assert_allclose(st, r_st, rtol=0, atol=1e-11)


def pin_stepwise_conv_equals_full_conv():
    """Stepwise updates from a zero conv state equal the full causal convolution of
    the sequence with K-1 zero left padding (np.convolve), for several K. The V
    channels carry silu(conv) unchanged."""
    for K in (2, 3, 4, 5):
        sh = Shape(batch=2, conv_kernel=K)
        T = 9
        x = draw(sh, T, 20 + K)
        s = O.shape_of(sh)
        cs = np.zeros((sh.batch, K - 1, sh.channels))
        v0 = 2 * sh.num_k_heads * sh.head_k_dim
        for t in range(T):
            act = O.conv_update(s, cs, x["qkv"][:, t], x["conv_w"])
            for b in range(sh.batch):
                for c in range(v0, sh.channels):
                    seq = x["qkv"][b, :, c].astype(np.float64)
                    u = np.convolve(seq, x["conv_w"][c, ::-1].astype(np.float64))[t]
                    assert abs(act[b, c] - u * expit(u)) <= 1e-13, (K, t, b, c)


def pin_conv_state_roll():
    """After one step the conv state is (old rows 1.., new input); after T >= K-1
    steps it holds exactly the last K-1 inputs, oldest first."""
    sh = Shape(conv_kernel=4)
    x = draw(sh, 6, 31)
    s = O.shape_of(sh)
    cs = x["conv_state"].astype(np.float64)
    old = cs.copy()
    O.conv_update(s, cs, x["qkv"][:, 0], x["conv_w"])
    np.testing.assert_array_equal(cs[:, :2], old[:, 1:])
    np.testing.assert_array_equal(cs[:, 2], x["qkv"][:, 0].astype(np.float64))
    for t in range(1, 6):
        O.conv_update(s, cs, x["qkv"][:, t], x["conv_w"])
    np.testing.assert_array_equal(cs, x["qkv"][:, 3:6].astype(np.float64))


def pin_identity_tap():
    """conv_w = e_{K-1} makes the conv the identity on the current token:
    V channels = silu(x) (scipy expit), Q/K = silu(x) scaled to norm sqrt(S/(S+eps))."""
    sh = Shape(l2_eps=1e-2)
    K, C = sh.conv_kernel, sh.channels
    x = draw(sh, 1, 41)
    w = np.zeros((C, K), dtype=np.float32)
    w[:, K - 1] = 1
    s = O.shape_of(sh)
    cs = x["conv_state"].astype(np.float64)
    act = O.conv_update(s, cs, x["qkv"][:, 0], w)
    xs = x["qkv"][:, 0].astype(np.float64)
    silu = xs * expit(xs)
    v0 = 2 * sh.num_k_heads * sh.head_k_dim
    np.testing.assert_allclose(act[:, v0:], silu[:, v0:], rtol=1e-15, atol=0)
    dk = sh.head_k_dim
    for b in range(sh.batch):
        for hd in range(2 * sh.num_k_heads):
            seg = slice(hd * dk, (hd + 1) * dk)
            S = float(np.sum(silu[b, seg] ** 2))
            np.testing.assert_allclose(np.sum(act[b, seg] ** 2), S / (S + sh.l2_eps), rtol=1e-13)
            # direction: parallel to silu(x) with a positive factor
            np.testing.assert_allclose(act[b, seg] / math.sqrt(np.sum(act[b, seg] ** 2)),
                                       silu[b, seg] / math.sqrt(S), rtol=0, atol=1e-14)


def pin_split_offsets():
    """Q | K | V split: a single nonzero input channel reaches exactly the head and
    position the split assigns (Q of k-head g at g*d_k, K at H_k*d_k + g*d_k, V of
    v-head h at 2*H_k*d_k + h*d_v); the readout of v-head h uses k-head h // G."""
    sh = Shape(batch=1)
    Hk, Hv, dk, dv, K, C = sh.num_k_heads, sh.num_v_heads, sh.head_k_dim, sh.head_v_dim, sh.conv_kernel, sh.channels
    s = O.shape_of(sh)
    w = np.zeros((C, K), dtype=np.float32)
    w[:, K - 1] = 1
    for c in (0, dk - 1, dk, Hk * dk, Hk * dk + dk + 3, 2 * Hk * dk, 2 * Hk * dk + dv, C - 1):
        q = np.zeros((1, C), dtype=np.float32)
        q[0, c] = 2.0
        act = O.conv_update(s, np.zeros((1, K - 1, C)), q, w)
        nz = np.nonzero(act[0])[0]
        assert list(nz) == [c], (c, nz)
    # k-head sharing: a state whose only nonzero row pattern lives in v-head h is read
    # with q of k-head h // G. Put q only in k-head g, then exactly the v-heads
    # g*G .. g*G+G-1 produce a nonzero readout.
    G = sh.group
    for g in range(Hk):
        act = np.zeros((1, C))
        act[0, g * dk] = 1.0  # q of k-head g = e_0
        st = np.ones((1, Hv, dk, dv))
        o, _, _ = O.recurrent_step(s, st, act, np.zeros((1, Hv), np.float32), np.full((1, Hv), -np.inf, np.float32),
                                   np.zeros(Hv, np.float32), np.zeros(Hv, np.float32))
        heads = sorted(set(np.nonzero(o[0])[0]))
        assert heads == list(range(g * G, (g + 1) * G)), (g, heads)


def pin_gate_closed_forms():
    """softplus(0) = ln 2; A_log = 0 gives alpha = sigmoid(-x); beta = sigmoid(b);
    both in (0, 1); b = +-inf gives beta = 1 / 0; A_log = -inf gives alpha = 1."""
    sh = Shape(batch=1, num_k_heads=1, num_v_heads=6, head_k_dim=4, head_v_dim=4)
    s = O.shape_of(sh)
    Hv = sh.num_v_heads
    zero_act = np.zeros((1, sh.channels))
    st = np.zeros((1, Hv, 4, 4))
    dt_bias = np.array([0.5, -1.25, 0.0, 2.0, -0.0625, 3.5], np.float32)
    A_log = np.array([0.0, 0.0, 1.0, math.log(3.0), 0.0, -2.0], np.float32)
    # x = 0 exactly: alpha = 2^-exp(A_log)
    _, al, be = O.recurrent_step(s, st, zero_act, (-dt_bias)[None], np.zeros((1, Hv), np.float32), A_log, dt_bias)
    np.testing.assert_allclose(al[0], 2.0 ** (-np.exp(A_log.astype(np.float64))), rtol=1e-15)
    np.testing.assert_array_equal(be[0], np.full(Hv, 0.5))
    # A_log = 0: alpha = sigmoid(-x)
    xr = np.linspace(-30, 30, Hv).astype(np.float32)
    bb = np.linspace(-8, 8, Hv).astype(np.float32)
    _, al, be = O.recurrent_step(s, st, zero_act, xr[None], bb[None], np.zeros(Hv, np.float32),
                                 np.zeros(Hv, np.float32))
    np.testing.assert_allclose(al[0], expit(-xr.astype(np.float64)), rtol=1e-13)
    np.testing.assert_allclose(be[0], expit(bb.astype(np.float64)), rtol=1e-15)
    assert np.all((al > 0) & (al < 1)) and np.all((be > 0) & (be < 1))
    _, al, be = O.recurrent_step(s, st, zero_act, xr[None], np.array([[np.inf, -np.inf] * 3], np.float32),
                                 np.full(Hv, -np.inf, np.float32), np.zeros(Hv, np.float32))
    np.testing.assert_array_equal(al[0], np.ones(Hv))
    np.testing.assert_array_equal(be[0], np.array([1.0, 0.0] * 3))


def _act_vector(sh, qs, ks, vs):
    """qkv_act for one sequence from per-k-head q, k and per-v-head v lists."""
    return np.concatenate([np.concatenate(qs), np.concatenate(ks), np.concatenate(vs)])[None]


def pin_unit_key_recall():
    """alpha = beta = 1 and a unit key k: after one step the state returns v for k
    (S k = v), whatever it held before; read out with q = k this is v / sqrt(d_k)."""
    sh = Shape(batch=1, num_k_heads=2, num_v_heads=4, head_k_dim=8, head_v_dim=6)
    s = O.shape_of(sh)
    rng = np.random.default_rng(51)
    Hk, Hv, dk, dv = sh.num_k_heads, sh.num_v_heads, sh.head_k_dim, sh.head_v_dim
    ks = [rng.standard_normal(dk) for _ in range(Hk)]
    ks = [k / np.linalg.norm(k) for k in ks]
    vs = [rng.standard_normal(dv) for _ in range(Hv)]
    act = _act_vector(sh, ks, ks, vs)
    st = rng.standard_normal((1, Hv, dk, dv))
    one = np.full((1, Hv), np.inf, np.float32)
    o, al, be = O.recurrent_step(s, st, act, np.zeros((1, Hv), np.float32), one,
                                 np.full(Hv, -np.inf, np.float32), np.zeros(Hv, np.float32))
    assert np.all(al == 1) and np.all(be == 1)
    for h in range(Hv):
        k = ks[h // sh.group]
        np.testing.assert_allclose(st[0, h].T @ k, vs[h], rtol=0, atol=1e-14)
        np.testing.assert_allclose(o[0, h], vs[h] / math.sqrt(dk), rtol=0, atol=1e-14)


def pin_orthonormal_keys():
    """alpha = beta = 1, keys e_0 .. e_{d_k-1} written in turn with values v_i into a
    zero state; querying e_i afterwards returns v_i / sqrt(d_k)."""
    sh = Shape(batch=1, num_k_heads=1, num_v_heads=1, head_k_dim=5, head_v_dim=3)
    s = O.shape_of(sh)
    dk, dv = sh.head_k_dim, sh.head_v_dim
    rng = np.random.default_rng(61)
    vals = rng.standard_normal((dk, dv))
    st = np.zeros((1, 1, dk, dv))
    inf1 = np.full((1, 1), np.inf, np.float32)
    for i in range(dk):
        e = np.eye(dk)[i]
        O.recurrent_step(s, st, _act_vector(sh, [e], [e], [vals[i]]), np.zeros((1, 1), np.float32), inf1,
                         np.full(1, -np.inf, np.float32), np.zeros(1, np.float32))
    for i in range(dk):
        e = np.eye(dk)[i]
        # beta = 0 keeps the state, so this is a pure read
        o, _, _ = O.recurrent_step(s, st.copy(), _act_vector(sh, [e], [e], [np.zeros(dv)]),
                                   np.zeros((1, 1), np.float32), -inf1, np.full(1, -np.inf, np.float32),
                                   np.zeros(1, np.float32))
        np.testing.assert_allclose(o[0, 0], vals[i] / math.sqrt(dk), rtol=0, atol=1e-15)


def pin_beta_zero_and_alpha_zero():
    """beta = 0: the state only decays, H' = alpha H. alpha -> 0: the past is
    forgotten, H' = k (beta v)^T."""
    sh = Shape(batch=1)
    s = O.shape_of(sh)
    Hk, Hv, dk, dv, G = sh.num_k_heads, sh.num_v_heads, sh.head_k_dim, sh.head_v_dim, sh.group
    rng = np.random.default_rng(71)
    ks = [rng.standard_normal(dk) for _ in range(Hk)]
    ks = [k / np.linalg.norm(k) for k in ks]
    qs = [rng.standard_normal(dk) for _ in range(Hk)]
    vs = [rng.standard_normal(dv) for _ in range(Hv)]
    act = _act_vector(sh, qs, ks, vs)
    st0 = rng.standard_normal((1, Hv, dk, dv))
    dt = rng.standard_normal((1, Hv)).astype(np.float32)
    A_log = rng.uniform(0, 2, Hv).astype(np.float32)
    st = st0.copy()
    _, al, be = O.recurrent_step(s, st, act, dt, np.full((1, Hv), -np.inf, np.float32), A_log,
                                 np.zeros(Hv, np.float32))
    assert np.all(be == 0)
    np.testing.assert_allclose(st, al[0][None, :, None, None] * st0, rtol=1e-15, atol=0)
    st = st0.copy()
    bb = rng.standard_normal((1, Hv)).astype(np.float32)
    _, al, be = O.recurrent_step(s, st, act, np.full((1, Hv), 200.0, np.float32), bb,
                                 np.full(Hv, 6.0, np.float32), np.zeros(Hv, np.float32))
    assert np.all(al == 0)
    for h in range(Hv):
        np.testing.assert_allclose(st[0, h], np.outer(ks[h // G], be[0, h] * vs[h]), rtol=1e-15, atol=1e-300)


def pin_exact_rationals():
    """Tiny heads with dyadic rational q, k, v (k not unit), beta = 1/2 exactly
    (b = 0) and alpha = 1/2 (A_log = 0, dt = -dt_bias), over 4 steps: the oracle
    equals exact rational arithmetic of S <- alpha S (I - beta k k^T) + beta v k^T,
    o = S q / sqrt(d_k), to 1e-14 relative."""
    sh = Shape(batch=1, num_k_heads=1, num_v_heads=2, head_k_dim=3, head_v_dim=2)
    s = O.shape_of(sh)
    rng = np.random.default_rng(81)
    dk, dv, Hv = 3, 2, 2
    S = [[[Fraction(int(rng.integers(-8, 9)), 8) for _ in range(dk)] for _ in range(dv)] for _ in range(Hv)]
    st = np.array([[[[float(S[h][j][i]) for j in range(dv)] for i in range(dk)] for h in range(Hv)]])
    half = Fraction(1, 2)
    dt_bias = np.float32(0.75)
    for step in range(4):
        q = [Fraction(int(rng.integers(-4, 5)), 4) for _ in range(dk)]
        k = [Fraction(int(rng.integers(-4, 5)), 4) for _ in range(dk)]
        vv = [[Fraction(int(rng.integers(-4, 5)), 4) for _ in range(dv)] for _ in range(Hv)]
        act = np.array([[float(t) for t in q + k + vv[0] + vv[1]]])
        o, al, be = O.recurrent_step(s, st, act, np.full((1, Hv), -dt_bias, np.float32), np.zeros((1, Hv), np.float32),
                                     np.zeros(Hv, np.float32), np.full(Hv, dt_bias, np.float32))
        assert be[0, 0] == 0.5 and abs(al[0, 0] - 0.5) < 1e-15
        for h in range(Hv):
            # S (I - beta k k^T) = S - beta (S k) k^T
            Sk = [sum(S[h][j][i] * k[i] for i in range(dk)) for j in range(dv)]
            S[h] = [[half * (S[h][j][i] - half * Sk[j] * k[i]) + half * vv[h][j] * k[i] for i in range(dk)]
                    for j in range(dv)]
            for j in range(dv):
                oj = sum(S[h][j][i] * q[i] for i in range(dk))
                exact = float(oj) / math.sqrt(dk)
                assert abs(o[0, h, j] - exact) <= 1e-14 * max(1.0, abs(exact)), (step, h, j)
                for i in range(dk):
                    assert abs(st[0, h, i, j] - float(S[h][j][i])) <= 1e-14 * max(1.0, abs(float(S[h][j][i])))


def pin_gated_norm():
    """Per-head RMSNorm and the silu(z) gate equal torch's rms_norm * silu; with
    w = 1 the normalised head has mean square m / (m + eps)."""
    sh = Shape(batch=2, rms_eps=1e-3)
    s = O.shape_of(sh)
    rng = np.random.default_rng(91)
    B, Hv, dv = sh.batch, sh.num_v_heads, sh.head_v_dim
    o = 0.05 * rng.standard_normal((B, Hv, dv))
    z = rng.standard_normal((B, Hv * dv)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    yn, out = O.gated_rmsnorm(s, o, z, w)
    ref = F.rms_norm(torch.from_numpy(o), (dv,), weight=torch.from_numpy(w.astype(np.float64)), eps=sh.rms_eps)
    np.testing.assert_allclose(yn, ref.numpy().reshape(B, -1), rtol=1e-14, atol=0)
    np.testing.assert_allclose(out, (ref * F.silu(torch.from_numpy(z.astype(np.float64)).reshape(B, Hv, dv))
                                     ).numpy().reshape(B, -1), rtol=1e-14, atol=1e-300)
    yn, _ = O.gated_rmsnorm(s, o, z, np.ones(dv, np.float32))
    m = np.mean(o ** 2, axis=-1)
    np.testing.assert_allclose(np.mean(yn.reshape(B, Hv, dv) ** 2, axis=-1), m / (m + sh.rms_eps), rtol=1e-13)


def pin_resume_and_decode_equivalence():
    """T1 steps then T2 steps equal T1 + T2 steps bitwise; T single decode steps
    equal one T-token sequence bitwise."""
    sh = Shape()
    T1, T2 = 3, 4
    x = draw(sh, T1 + T2, 101)
    full, cs_f, st_f = run_oracle(sh, x, T1 + T2)
    s = O.shape_of(sh)
    cs = x["conv_state"].astype(np.float64)
    st = x["state"].astype(np.float64)
    parts = []
    for lo, hi in ((0, T1), (T1, T1 + T2)):
        sl = lambda a: np.ascontiguousarray(a[:, lo:hi])
        parts.append(O.sequence(s, hi - lo, cs, st, sl(x["qkv"]), x["conv_w"], sl(x["a"]), sl(x["b"]),
                                sl(x["z"]), x["A_log"], x["dt_bias"], x["norm_w"]))
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), full)
    np.testing.assert_array_equal(cs, cs_f)
    np.testing.assert_array_equal(st, st_f)
    cs = x["conv_state"].astype(np.float64)
    st = x["state"].astype(np.float64)
    for t in range(T1 + T2):
        o = O.decode_step(s, cs, st, x["qkv"][:, t], x["conv_w"], x["a"][:, t], x["b"][:, t], x["z"][:, t],
                          x["A_log"], x["dt_bias"], x["norm_w"])
        np.testing.assert_array_equal(o, full[:, t])


def pin_permutation_equivariance():
    """Permuting sequences permutes outputs; permuting k-head groups (their Q, K
    channels, their v-heads' V channels, states, gates, z) permutes outputs."""
    sh = Shape(batch=3, num_k_heads=3, num_v_heads=6)
    T = 3
    x = draw(sh, T, 111)
    out, cs, st = run_oracle(sh, x, T)
    perm = np.array([2, 0, 1])
    xp = {k_: (v_[perm] if k_ in ("state", "conv_state", "qkv", "z", "a", "b") else v_) for k_, v_ in x.items()}
    out_p, cs_p, st_p = run_oracle(sh, xp, T)
    np.testing.assert_array_equal(out_p, out[perm])
    np.testing.assert_array_equal(st_p, st[perm])
    Hk, Hv, dk, dv, G = sh.num_k_heads, sh.num_v_heads, sh.head_k_dim, sh.head_v_dim, sh.group
    gp = np.array([1, 2, 0])
    hp = np.concatenate([np.arange(g * G, (g + 1) * G) for g in gp])
    ch = np.concatenate([np.arange(g * dk, (g + 1) * dk) for g in gp] +
                        [Hk * dk + np.arange(g * dk, (g + 1) * dk) for g in gp] +
                        [2 * Hk * dk + np.arange(h * dv, (h + 1) * dv) for h in hp])
    zc = np.concatenate([np.arange(h * dv, (h + 1) * dv) for h in hp])
    xg = dict(x)
    xg["conv_w"] = x["conv_w"][ch]
    xg["conv_state"] = x["conv_state"][:, :, ch]
    xg["qkv"] = x["qkv"][:, :, ch]
    xg["state"] = x["state"][:, hp]
    xg["A_log"], xg["dt_bias"] = x["A_log"][hp], x["dt_bias"][hp]
    xg["a"], xg["b"] = x["a"][:, :, hp], x["b"][:, :, hp]
    xg["z"] = x["z"][:, :, zc]
    out_g, cs_g, st_g = run_oracle(sh, xg, T)
    np.testing.assert_array_equal(out_g, out[:, :, zc])
    np.testing.assert_array_equal(st_g, st[:, hp])
    np.testing.assert_array_equal(cs_g, cs[:, :, ch])


def pin_linear_projection():
    """The projections (step 2 and steps 9-11 of "linear_attention.rs") as
    y[m][n] = sum_k x[m][k] w[n][k]: identity weights give x back exactly; all-ones x
    with integer weights w[n][k] = n + k gives the exact sums K n + K (K - 1) / 2; a
    rectangular random case equals numpy's float64 matrix product of the same values to
    rounding, and swapping the roles of x and w transposes the result."""
    rng = np.random.default_rng(7)
    K = 24
    x = rng.standard_normal((3, K)).astype(np.float32)
    np.testing.assert_array_equal(O.linear(x, np.eye(K, dtype=np.float32)), x.astype(np.float64))
    N = 5
    w = (np.arange(N)[:, None] + np.arange(K)[None, :]).astype(np.float32)
    y = O.linear(np.ones((1, K), dtype=np.float32), w)
    np.testing.assert_array_equal(y[0], K * np.arange(N) + K * (K - 1) / 2)
    M, N, K = 4, 7, 33
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    y = O.linear(x, w)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(O.linear(w, x), y.T)


ALL_PINS = [
    pin_library_composition,
    pin_stepwise_conv_equals_full_conv,
    pin_conv_state_roll,
    pin_identity_tap,
    pin_split_offsets,
    pin_gate_closed_forms,
    pin_unit_key_recall,
    pin_orthonormal_keys,
    pin_beta_zero_and_alpha_zero,
    pin_exact_rationals,
    pin_gated_norm,
    pin_resume_and_decode_equivalence,
    pin_permutation_equivariance,
    pin_linear_projection,
]
