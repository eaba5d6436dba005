"""The seeded input generators: deterministic, the stated distributions, and an exact
bf16 conversion (checked against torch's round-to-nearest-even)."""

import hashlib
import math

import numpy as np
import pytest
import torch

from gated_deltanet_linear_causal_amd import inputs as I


def _digest(d):
    h = hashlib.sha256()
    for k in sorted(d):
        h.update(k.encode())
        h.update(np.ascontiguousarray(d[k]).tobytes())
    return h.hexdigest()


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40], np.float32)])
    ours = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = I.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_configs_shapes():
    c = I.CONFIGS
    assert [x.seed for x in c] == [0, 1, 2, 3, 4]
    assert c[0].channels == 192 and c[0].act_dtype == "f32" and c[0].steps == 16
    for x in c[1:]:
        assert (x.num_k_heads, x.num_v_heads, x.head_k_dim, x.head_v_dim, x.conv_kernel) == (16, 32, 128, 128, 4)
        assert x.channels == 8192 and x.z_dim == 4096 and x.group == 2
    assert [x.batch for x in c[1:]] == [1, 64, 512, 8]
    assert c[4].mode == "sequence" and c[4].steps == 4096


@pytest.mark.parametrize("i", [0, 1])
def test_deterministic(i):
    cfg = I.config(i)
    assert _digest(I.generate(cfg)) == _digest(I.generate(cfg))
    assert _digest(I.generate(cfg)) != _digest(I.generate(cfg.with_(seed=cfg.seed + 100)))


def test_distributions_qwen35():
    cfg = I.config(1).with_(batch=4)
    d = I.generate(cfg, steps=8)
    q = I.widen(d["qkv"], "bf16")
    assert abs(q.mean()) < 0.01 and abs(q.std() - 1) < 0.01
    w = I.widen(d["conv_w"], "bf16")
    assert abs(w.std() - 0.5) < 0.01
    assert abs(d["state"].std() - 0.02) < 2e-4
    cs = I.widen(d["conv_state"], "bf16")
    assert abs(cs.std() - 1) < 0.01
    assert d["A_log"].min() >= 0 and d["A_log"].max() <= math.log(16)
    sp = np.log1p(np.exp(d["dt_bias"].astype(np.float64)))  # softplus(dt_bias) = u
    assert sp.min() >= 1e-3 * 0.999 and sp.max() <= 0.1 * 1.001
    assert abs(d["norm_w"].mean() - 1) < 0.05
    assert d["qkv"].dtype == np.uint16 and d["state"].dtype == np.float32


def test_tiny_config_zero_states():
    d = I.generate(I.config(0))
    assert not d["state"].any() and not d["conv_state"].any()
    assert d["qkv"].shape == (16, 1, 192) and d["z"].shape == (16, 1, 64) and d["a"].shape == (16, 1, 2)
    assert d["qkv"].dtype == np.float32
