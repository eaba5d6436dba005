"""The chunked form of the delta rule, modelled in fp64 on the CPU (chunk_model.py),
against the sequential fp64 oracle: T tokens in chunks of C in {1, 4, 32, 64} must give
the oracle's per-token readouts and final state to 1e-12, with the last chunk ragged,
for the three ways of solving for Delta, with k-heads shared by two v-heads, d_k != d_v,
and gates whose running log sum falls far below the fp64 range inside a chunk. Likewise
the unrolled form the speculative verification evaluates draft tokens in (deltas and
readouts from the state before the draft), and the commit's replay of its updates.

The pages give only the per-token rule (page "linear_attention.rs", step 7); the
chunked regrouping is derived from it, so this is the check of that derivation that
runs before any GPU code: the HIP chunk kernel implements the "inverse" form."""

import numpy as np
import pytest

from gated_deltanet_linear_causal_amd import inputs as I
from oracle import oracle as O

import chunk_model as M


def _case(T=100, dk=16, dv=24, seed=11, strong_decay=False):
    cfg = I.GdnConfig(name="chunk_model", batch=2, num_k_heads=2, num_v_heads=4, head_k_dim=dk, head_v_dim=dv,
                      conv_kernel=4, act_dtype="f32", steps=T, seed=seed, mode="sequence", state_std=0.3,
                      conv_state_std=1.0)
    data = I.generate(cfg)
    if strong_decay:
        # dt = +30 on every token: log alpha = -exp(A_log) softplus(30 + dt_bias), between
        # -30 and -480 per token, so g falls to ~ -15000 within a chunk of 32 and exp(g)
        # is 0 in fp64 for most tokens; alpha itself stays a normal fp64 number.
        # Every third token keeps its drawn dt, so the decay is not uniform.
        a = data["a"].copy()
        a[:, 1::3] = 30.0
        a[:, 2::3] = 30.0
        data["a"] = a
    return cfg, data


def _oracle_by_token(cfg, data, states=None):
    """Per-token q, k, v (after conv, SiLU and the L2 norms), alpha, beta and readout o
    of every (sequence, v-head), and the final state, from the oracle's step functions.
    `states`, a list, receives the state after each token."""
    s = O.shape_of(cfg)
    B, T, Hk, Hv, dk, dv = cfg.batch, cfg.steps, cfg.num_k_heads, cfg.num_v_heads, cfg.head_k_dim, cfg.head_v_dim
    G = Hv // Hk
    cs = data["conv_state"].astype(np.float64)
    st = data["state"].astype(np.float64)
    q = np.zeros((B, Hv, T, dk))
    k = np.zeros((B, Hv, T, dk))
    v = np.zeros((B, Hv, T, dv))
    o = np.zeros((B, Hv, T, dv))
    alpha = np.zeros((B, Hv, T))
    beta = np.zeros((B, Hv, T))
    for t in range(T):
        act = O.conv_update(s, cs, data["qkv"][:, t], data["conv_w"])
        for h in range(Hv):
            g = h // G
            q[:, h, t] = act[:, g * dk:(g + 1) * dk]
            k[:, h, t] = act[:, (Hk + g) * dk:(Hk + g + 1) * dk]
            v[:, h, t] = act[:, 2 * Hk * dk + h * dv:2 * Hk * dk + (h + 1) * dv]
        ot, at, bt = O.recurrent_step(s, st, act, data["a"][:, t], data["b"][:, t], data["A_log"], data["dt_bias"])
        o[:, :, t], alpha[:, :, t], beta[:, :, t] = ot, at, bt
        if states is not None:
            states.append(st.copy())
    return q, k, v, o, alpha, beta, st


@pytest.fixture(scope="module", params=[False, True], ids=["drawn_gates", "strong_decay"])
def case(request):
    cfg, data = _case(strong_decay=request.param)
    return cfg, data, _oracle_by_token(cfg, data)


def _gates(cfg, data):
    dt = data["a"].astype(np.float64)                    # [B][T][H_v]
    la = M.log_alpha(dt, data["dt_bias"].astype(np.float64), data["A_log"].astype(np.float64))
    beta = M.sigmoid(data["b"].astype(np.float64))
    return np.transpose(la, (0, 2, 1)), np.transpose(beta, (0, 2, 1))   # [B][H_v][T]


def test_gate_inputs_match_the_oracle(case):
    cfg, data, (q, k, v, o, alpha, beta, st) = case
    la, bt = _gates(cfg, data)
    np.testing.assert_allclose(np.exp(la), alpha, rtol=1e-13, atol=0)
    np.testing.assert_allclose(bt, beta, rtol=1e-14, atol=0)


@pytest.mark.parametrize("chunk", [1, 4, 32, 64])
@pytest.mark.parametrize("form", ["solve", "wy", "inverse"])
def test_chunked_equals_sequential(case, chunk, form):
    cfg, data, (q, k, v, o, alpha, beta, st) = case
    la, bt = _gates(cfg, data)
    H0 = data["state"].astype(np.float64)
    worst_o = worst_h = 0.0
    for b in range(cfg.batch):
        for h in range(cfg.num_v_heads):
            om, hm = M.sequence(H0[b, h], q[b, h], k[b, h], v[b, h], la[b, h], bt[b, h], chunk, form)
            assert np.all(np.isfinite(om)) and np.all(np.isfinite(hm))
            worst_o = max(worst_o, float(np.abs(om - o[b, h]).max() / max(1.0, np.abs(o[b, h]).max())))
            worst_h = max(worst_h, float(np.abs(hm - st[b, h]).max() / max(1.0, np.abs(st[b, h]).max())))
    print("C=%d %s: readout %.2e, state %.2e" % (chunk, form, worst_o, worst_h))
    assert worst_o <= 1e-12 and worst_h <= 1e-12


def test_strong_decay_really_underflows():
    """The strong-decay case does reach the regime it is meant to cover: inside a chunk
    of 32 the running log-gate sum passes -745, where exp(g) is 0 in fp64."""
    cfg, data = _case(strong_decay=True)
    la, _ = _gates(cfg, data)
    g = np.cumsum(la[..., :32], axis=-1)
    assert g.min() < -745.0 and np.exp(g.min()) == 0.0


def test_blocked_inverse_is_the_inverse():
    rng = np.random.default_rng(5)
    for n in (1, 2, 7, 32):
        A = np.tril(rng.uniform(-1, 1, (n, n)), -1)
        T = M.blocked_inverse(A)
        np.testing.assert_allclose(T @ (np.eye(n) + A), np.eye(n), atol=1e-12)
        assert np.array_equal(np.triu(T, 1), np.zeros((n, n)))


def test_model_catches_a_planted_mistake():
    """The comparison has teeth: dropping the decay of H0 in the state update (gamma_C
    taken as 1) is caught far above the 1e-12 bound."""
    cfg, data = _case(T=40)
    q, k, v, o, alpha, beta, st = _oracle_by_token(cfg, data)
    la, bt = _gates(cfg, data)
    H0 = data["state"].astype(np.float64)

    saved = M.chunk_step

    def bad_step(H, Q, K, V, l, b, form="solve"):
        O_, Hn = saved(H, Q, K, V, l, b, form)
        return O_, Hn + (1.0 - np.exp(np.sum(l))) * H

    try:
        M.chunk_step = bad_step
        om, hm = M.sequence(H0[0, 0], q[0, 0], k[0, 0], v[0, 0], la[0, 0], bt[0, 0], 4)
    finally:
        M.chunk_step = saved
    assert np.abs(hm - st[0, 0]).max() > 1e-3


@pytest.fixture(scope="module", params=[False, True], ids=["drawn_gates", "strong_decay"])
def draft_case(request):
    cfg, data = _case(T=8, strong_decay=request.param)
    states = []
    return cfg, data, _oracle_by_token(cfg, data, states), states


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_draft_unrolled_equals_sequential(draft_case, T):
    """The draft tokens' readouts from H0 alone equal the oracle's token-by-token ones,
    and replaying the recorded deltas gives the oracle's state after every prefix."""
    cfg, data, (q, k, v, o, alpha, beta, st), states = draft_case
    H0 = data["state"].astype(np.float64)
    worst_o = worst_h = 0.0
    for b in range(cfg.batch):
        for h in range(cfg.num_v_heads):
            D, om = M.draft_unrolled(H0[b, h], q[b, h, :T], k[b, h, :T], v[b, h, :T], alpha[b, h, :T], beta[b, h, :T])
            assert np.all(np.isfinite(om)) and np.all(np.isfinite(D))
            worst_o = max(worst_o, float(np.abs(om - o[b, h, :T]).max() / max(1.0, np.abs(o[b, h, :T]).max())))
            for n in range(T + 1):
                ref = H0[b, h] if n == 0 else states[n - 1][b, h]
                hm = M.replay(H0[b, h], k[b, h], D, alpha[b, h], n)
                worst_h = max(worst_h, float(np.abs(hm - ref).max() / max(1.0, np.abs(ref).max())))
    print("T=%d: readout %.2e, replayed states %.2e" % (T, worst_o, worst_h))
    assert worst_o <= 1e-12 and worst_h <= 1e-12


def test_draft_model_catches_a_planted_mistake(draft_case):
    """An off-by-one in the decay products (G(s, t-1) for G(s+1, t-1)) is caught."""
    cfg, data, (q, k, v, o, alpha, beta, st), _ = draft_case
    H0 = data["state"].astype(np.float64)
    _, om = M.draft_unrolled(H0[0, 0], q[0, 0], k[0, 0], v[0, 0], alpha[0, 0], beta[0, 0], shift=0)
    err = float(np.abs(om - o[0, 0]).max() / max(1.0, np.abs(o[0, 0]).max()))
    print("planted: readout %.2e" % err)
    assert err > 1e-6

