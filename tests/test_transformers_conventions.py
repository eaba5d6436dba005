"""The layer conventions the pages leave open, checked against an independent
implementation: the PyTorch reference of the Qwen3.5 gated-delta-net layer shipped in
`transformers` (`models/qwen3_5`). The oracle was written from the pages alone; this
test ties the readings below to that implementation, on tiny fp32 shapes, on the CPU.

* R1, state orientation: H[i in d_k][j in d_v], readout sum_i H[i][j] q_i / sqrt(d_k);
* R2, conv taps and state rows: tap K-1 on the current token, row 0 the oldest,
  weights [C][K];
* R4, L2 norm x / sqrt(sum x^2 + eps) of q and k per head;
* R6, R7, per-head RMSNorm with the plain weight w, then the silu(z) gate;
* R9, v-head h reads k-head floor(h / G);
* the Q | K | V order of the channel axis and the gates
  alpha = exp(-exp(A_log) softplus(dt + dt_bias)), beta = sigmoid(b)
  ("linear_attention.rs", steps 3-11).

`transformers` evaluates the delta rule in fp32, so the bound is 1e-4 relative: a
convention that differs moves the results by O(1). The test is skipped if the module
is not importable."""

import types

import numpy as np
import pytest

torch = pytest.importorskip("torch")
q35 = pytest.importorskip("transformers.models.qwen3_5.modeling_qwen3_5")

from gated_deltanet_linear_causal_amd import inputs as I
from oracle import oracle as O

B, HK, HV, DK, DV, K, HID = 2, 2, 4, 16, 24, 4, 32
G = HV // HK
C = 2 * HK * DK + HV * DV
TOL = 1e-4


def _cfg(T):
    return I.GdnConfig(name="transformers_pin", batch=B, num_k_heads=HK, num_v_heads=HV, head_k_dim=DK,
                       head_v_dim=DV, conv_kernel=K, act_dtype="f32", steps=T, seed=21, mode="sequence",
                       state_std=0.3, conv_state_std=1.0)


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(1e-30, np.abs(b).max()))


def _f32(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def test_layer_forward_matches_transformers():
    """The whole layer, from zero states (the module's prefill path with no cache):
    in_proj, conv, gates, delta rule, gated RMSNorm and out_proj against
    `Qwen3_5GatedDeltaNet.forward`."""
    T = 6
    cfg = _cfg(T)
    data = I.generate(cfg)
    rng = np.random.default_rng(7)
    x = _f32(rng, (B, T, HID))
    w_qkv, w_z = _f32(rng, (C, HID), HID ** -0.5), _f32(rng, (HV * DV, HID), HID ** -0.5)
    w_a, w_b = _f32(rng, (HV, HID), HID ** -0.5), _f32(rng, (HV, HID), HID ** -0.5)
    w_out = _f32(rng, (HID, HV * DV), (HV * DV) ** -0.5)

    # oracle: projections, then T steps of the layer from zero conv and recurrent states
    s = O.shape_of(cfg)
    xf = x.reshape(B * T, HID)
    lin = lambda w, n: O.linear(xf, w).reshape(B, T, n)
    out = O.sequence(s, T, np.zeros((B, K - 1, C)), np.zeros((B, HV, DK, DV)), lin(w_qkv, C), data["conv_w"],
                     lin(w_a, HV), lin(w_b, HV), lin(w_z, HV * DV), data["A_log"], data["dt_bias"], data["norm_w"])
    # the oracle's layer takes its inputs as fp32 values: so does the module here, after
    # the projections, to compare the same arithmetic
    y_oracle = O.linear(out.reshape(B * T, HV * DV).astype(np.float32), w_out).reshape(B, T, HID)

    conf = types.SimpleNamespace(hidden_size=HID, linear_num_value_heads=HV, linear_num_key_heads=HK,
                                 linear_key_head_dim=DK, linear_value_head_dim=DV, linear_conv_kernel_dim=K,
                                 hidden_act="silu", rms_norm_eps=cfg.rms_eps, layer_types=["linear_attention"])
    m = q35.Qwen3_5GatedDeltaNet(conf, 0).double()
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    with torch.no_grad():
        m.in_proj_qkv.weight.copy_(t(w_qkv))
        m.in_proj_z.weight.copy_(t(w_z))
        m.in_proj_a.weight.copy_(t(w_a))
        m.in_proj_b.weight.copy_(t(w_b))
        m.out_proj.weight.copy_(t(w_out))
        m.conv1d.weight.copy_(t(data["conv_w"])[:, None, :])
        m.A_log.copy_(t(data["A_log"]))
        m.dt_bias.copy_(t(data["dt_bias"]))
        m.norm.weight.copy_(t(data["norm_w"]))
        y_ref = m(t(x)).numpy()
    err = _rel(y_oracle, y_ref)
    print("layer forward: max rel %.2e" % err)
    assert np.all(np.isfinite(y_oracle)) and err <= TOL


def test_decode_steps_with_nonzero_states_match_transformers():
    """Decode steps from nonzero conv and recurrent states (where the row order of the
    conv state and the orientation of H matter): the conv update, the delta rule with
    its readout, and the gated RMSNorm against `causal_conv1d_update`,
    `torch_recurrent_gated_delta_rule` and `Qwen3_5RMSNormGated`."""
    T = 3
    cfg = _cfg(T)
    data = I.generate(cfg)
    s = O.shape_of(cfg)
    cs = data["conv_state"].astype(np.float64)       # [B][K-1][C], row 0 the oldest
    st = data["state"].astype(np.float64)            # [B][H_v][d_k][d_v]
    cs_ref = torch.from_numpy(np.ascontiguousarray(np.swapaxes(cs, 1, 2)))   # [B][C][K-1]
    st_ref = torch.from_numpy(st.copy())
    w = torch.from_numpy(data["conv_w"].astype(np.float64))
    norm = q35.Qwen3_5RMSNormGated(DV, eps=cfg.rms_eps).double()
    with torch.no_grad():
        norm.weight.copy_(torch.from_numpy(data["norm_w"].astype(np.float64)))
    worst = {}
    for step in range(T):
        qkv = data["qkv"][:, step]
        act = O.conv_update(s, cs, qkv, data["conv_w"])
        act_ref = q35.causal_conv1d_update(torch.from_numpy(qkv.astype(np.float64))[:, :, None], cs_ref, w, None,
                                           "silu")[:, :, 0].numpy()
        # the page's step 3 normalises q and k inside the conv update; the module does it
        # in the delta rule (use_qk_l2norm_in_kernel), with its own l2norm
        a64 = torch.from_numpy(act_ref)
        qk_unit = [q35.l2norm(a64[:, j * HK * DK:(j + 1) * HK * DK].reshape(B, HK, DK), dim=-1, eps=cfg.l2_eps)
                   .reshape(B, HK * DK).numpy() for j in (0, 1)]
        act_unit = np.concatenate(qk_unit + [act_ref[:, 2 * HK * DK:]], axis=1)
        worst["conv"] = max(worst.get("conv", 0.0), _rel(act, act_unit))
        worst["conv_state"] = max(worst.get("conv_state", 0.0), _rel(cs, np.swapaxes(cs_ref.numpy(), 1, 2)))

        o, alpha, beta = O.recurrent_step(s, st, act, data["a"][:, step], data["b"][:, step], data["A_log"],
                                          data["dt_bias"])
        q = a64[:, :HK * DK].reshape(B, 1, HK, DK).repeat_interleave(G, dim=2)
        k = a64[:, HK * DK:2 * HK * DK].reshape(B, 1, HK, DK).repeat_interleave(G, dim=2)
        v = a64[:, 2 * HK * DK:].reshape(B, 1, HV, DV)
        # the gates come from the oracle here (the forward test above checks them)
        g = torch.from_numpy(np.log(alpha))[:, None, :]
        bt = torch.from_numpy(beta)[:, None, :]
        o_ref, st_new = q35.torch_recurrent_gated_delta_rule(q, k, v, g=g, beta=bt, initial_state=st_ref,
                                                             output_final_state=True, use_qk_l2norm_in_kernel=True)
        st_ref = st_new.double()
        worst["readout"] = max(worst.get("readout", 0.0), _rel(o, o_ref[:, 0].numpy()))
        worst["state"] = max(worst.get("state", 0.0), _rel(st, st_ref.numpy()))

        z = data["z"][:, step]
        _, out = O.gated_rmsnorm(s, o, z, data["norm_w"])
        with torch.no_grad():
            out_ref = norm(torch.from_numpy(o.reshape(B * HV, DV)),
                           torch.from_numpy(z.astype(np.float64).reshape(B * HV, DV))).numpy()
        worst["gated_norm"] = max(worst.get("gated_norm", 0.0), _rel(out, out_ref.reshape(B, HV * DV)))
    print(" ".join("%s %.2e" % kv for kv in worst.items()))
    for name, err in worst.items():
        assert err <= TOL, (name, err)


def test_the_comparison_has_teeth():
    """A transposed state (the one convention R1 fixes) moves the readout far past the
    bound: the check above would catch an oracle that read H the other way round."""
    cfg = _cfg(1).with_(head_v_dim=DK)
    data = I.generate(cfg)
    s = O.shape_of(cfg)
    cs = data["conv_state"].astype(np.float64)
    st = data["state"].astype(np.float64)
    act = O.conv_update(s, cs, data["qkv"][:, 0], data["conv_w"])
    st_t = np.ascontiguousarray(np.swapaxes(st, 2, 3))
    o, alpha, beta = O.recurrent_step(s, st, act, data["a"][:, 0], data["b"][:, 0], data["A_log"], data["dt_bias"])
    o_t, _, _ = O.recurrent_step(s, st_t, act, data["a"][:, 0], data["b"][:, 0], data["A_log"], data["dt_bias"])
    assert _rel(o_t, o) > 100 * TOL
