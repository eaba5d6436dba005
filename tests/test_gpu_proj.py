"""The projections around the layer through the C-ABI (gdn_in_proj, gdn_out_proj)
against the fp64 oracle's y = x W^T on the same bf16 values.

Tolerance: the kernels accumulate in fp32 and round once to the output dtype.
* bf16 outputs: |got - ref| <= 2^-8 |ref| + 1e-5, i.e. the half-ulp of the final
  round-to-nearest-even plus slack for the fp32 sum (a result near a rounding
  boundary may land on the neighbouring bf16 value).
* fp32 outputs: 1e-5 absolute + 1e-5 relative. The weights are scaled by
  1/sqrt(fan_in), so outputs are O(1) and the fp32 sum of K <= 4096 products has an
  error of order sqrt(K) 2^-24, a few 1e-7.
Shapes cover every kernel: weight streaming (B <= 8, or B <= 2), the skinny MFMA kernel
(3..32 rows, few output columns: out_proj at B = 3 and 20, in_proj at hidden 512), the
register-staged 32 x 32 tiles (out_proj of the small layers at B = 9 and 100, in_proj at
B = 100), and the DMA-fed rings with 64-deep stages: 32 x 32 (in_proj at B = 3 and 20),
32 x 64 (in_proj at B = 33, 40 and 64, out_proj at B = 512 and 600, the 33, 40 and 600
with a ragged last row tile), 64 x 64 by 4 stages (in_proj at B = 128, out_proj at B =
1024), 64 x 128 by 3 stages (in_proj at B = 150 and 200, ragged), 64 x 64 by 3 stages
(in_proj at B = 300 and 600, ragged), 128 x 128 (in_proj of an H_k = 20, H_v = 40 layer
at B = 256) and 256 x 128 (in_proj at B = 512 and 1024); and with the 128-deep stages of
out_proj's 4096-long contraction: 16 x 16 tiles of one wave (B = 33, 40, 64 and 128), 32
x 16 (B = 150, ragged, and the narrow outputs of hidden 64..192) and 32 x 32 (B = 200
and 300, ragged); ragged row and column tiles (the H_v-wide a/b segments are narrower
than a tile) and the Qwen3.5-style sizes. The rings take their stages in a staggered
order per workgroup while the activations are at most 2 MB (most cases here) and in the
common order above that (in_proj at B = 600 and 1024, out_proj at B = 300, 512, 600,
1024). The ring kernels store their tiles in 16-byte pieces; a segment whose width is
not a multiple of 8 bf16 values (the a/b segments of the H_v = 20 layer at B = 1024) is
stored element by element.
"""

import numpy as np
import pytest
import torch

from gated_deltanet_linear_causal_amd import gdn
from gated_deltanet_linear_causal_amd import inputs as I
from oracle import oracle as O

from gdn_cases import dev, host_f64, shape_for

pytestmark = pytest.mark.gpu


def bf(a):
    return I.bf16_bits_to_f32(a)


def check_bf16(name, got, ref):
    got = host_f64(got)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5
    print("%-36s max_abs %.3e  worst err/bound %.3f" % (name, err.max(), (err / bound).max()))
    assert np.all(err <= bound), name


def check_f32(name, got, ref):
    got = host_f64(got)
    err = np.abs(got - ref)
    bound = 1e-5 + 1e-5 * np.abs(ref)
    print("%-36s max_abs %.3e  worst err/bound %.3f" % (name, err.max(), (err / bound).max()))
    assert np.all(err <= bound), name


def cfg_of(B, Hk=16, Hv=32, d=128):
    return I.GdnConfig(name="proj", batch=B, num_k_heads=Hk, num_v_heads=Hv, head_k_dim=d, head_v_dim=d,
                       conv_kernel=4, act_dtype="bf16", steps=1, seed=300 + B + Hv, mode="decode",
                       state_std=0.02, conv_state_std=1.0)


CASES = [
    # B, Hk, Hv, d, hidden, rows checked (None: all)
    (1, 16, 32, 128, 2048, None),
    (2, 16, 32, 128, 2048, None),
    (3, 16, 32, 128, 2048, None),
    (8, 2, 4, 64, 512, None),
    (9, 2, 4, 64, 512, None),
    (20, 16, 32, 128, 2048, None),
    (33, 16, 32, 128, 2048, None),
    (40, 16, 32, 128, 2048, None),
    (64, 16, 32, 128, 2048, None),
    (100, 2, 6, 64, 256, None),
    (128, 16, 32, 128, 2048, [0, 1, 15, 63, 64, 100, 127]),
    (150, 16, 32, 128, 2048, [0, 31, 32, 127, 128, 149]),
    (200, 16, 32, 128, 2048, [0, 1, 127, 128, 150, 199]),
    (300, 16, 32, 128, 2048, [0, 63, 64, 255, 256, 299]),
    (256, 20, 40, 128, 2048, [0, 1, 127, 128, 255]),
    (600, 16, 32, 128, 2048, [0, 63, 64, 511, 512, 575, 576, 599]),
    (512, 16, 32, 128, 2048, None),  # the benchmark's B = 512 shapes, every row
    (1024, 4, 20, 128, 2048, [0, 1, 255, 256, 511, 767, 1000, 1023]),
    # contractions of 1, 2 and 3 stages through the 256 x 128 ring (in_proj, hidden 64 /
    # 128 / 192) and of 1..4 stages through the 32 x 64 ring (out_proj, H_v d_v = 64 ..
    # 256): the prologue issues fewer stages than the ring holds and every stage is a tail
    (512, 16, 32, 128, 64, [0, 255, 256, 511]),
    (512, 16, 32, 128, 128, [0, 300, 511]),
    (512, 16, 32, 128, 192, [1, 256, 510]),
    (512, 1, 1, 64, 2048, [0, 255, 256, 511]),
    (512, 1, 2, 64, 2048, [0, 511]),
    (512, 1, 3, 64, 2048, [0, 511]),
    (512, 2, 4, 64, 2048, [0, 511]),
]


@pytest.mark.parametrize("case", CASES, ids=["B%d_Hv%d_d%d_h%d" % (c[0], c[2], c[3], c[4]) for c in CASES])
def test_in_and_out_projections(case):
    B, Hk, Hv, d, hidden, rows = case
    print("case B=%d Hk=%d Hv=%d d=%d hidden=%d" % (B, Hk, Hv, d, hidden), flush=True)
    cfg = cfg_of(B, Hk, Hv, d)
    P = I.generate_projections(cfg, hidden)
    x = dev(P["x_norm"], "bf16")
    w = {k: dev(P[k], "bf16") for k in ("w_qkv", "w_z", "w_a", "w_b", "w_out")}
    C, zd = cfg.channels, Hv * d
    s = shape_for(cfg)
    outs = {k: torch.full((B, n), float("nan"), dtype=torch.bfloat16, device="cuda")
            for k, n in (("qkv", C), ("z", zd), ("dt_raw", Hv), ("b_raw", Hv))}
    gdn.gdn_in_proj(s, hidden, x, w["w_qkv"], w["w_z"], w["w_a"], w["w_b"], outs["qkv"], outs["z"],
                    outs["dt_raw"], outs["b_raw"])
    # out_proj of a bf16 gated vector, fp32 and bf16 outputs
    g = I.f32_to_bf16_bits(np.random.default_rng(B).standard_normal((B, zd), dtype=np.float32))
    gd = dev(g, "bf16")
    y32 = torch.full((B, hidden), float("nan"), dtype=torch.float32, device="cuda")
    y16 = torch.full((B, hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_out_proj(s, hidden, gd, w["w_out"], y32)
    gdn.gdn_out_proj(shape_for(cfg, out_dtype="bf16"), hidden, gd, w["w_out"], y16)
    torch.cuda.synchronize()

    idx = np.arange(B) if rows is None else np.asarray(rows)
    xr = bf(P["x_norm"][idx])
    for k, wk in (("qkv", "w_qkv"), ("z", "w_z"), ("dt_raw", "w_a"), ("b_raw", "w_b")):
        ref = O.linear(xr, bf(P[wk]))
        check_bf16("in_proj %s" % k, outs[k][torch.as_tensor(idx, device="cuda")], ref)
    ref = O.linear(bf(g[idx]), bf(P["w_out"]))
    sel = torch.as_tensor(idx, device="cuda")
    check_f32("out_proj f32", y32[sel], ref)
    check_bf16("out_proj bf16", y16[sel], ref)


def test_projection_then_decode_layer():
    """The in_proj outputs are exactly the inputs gdn_decode_layer takes: running the
    layer on them gives the oracle's step on the same (bf16) values."""
    from gdn_cases import TOL, compare
    cfg = cfg_of(4)
    data = I.generate(cfg, steps=1)
    P = I.generate_projections(cfg)
    s = shape_for(cfg)
    B, C, Hv, zd = cfg.batch, cfg.channels, cfg.num_v_heads, cfg.z_dim
    qkv = torch.empty((B, C), dtype=torch.bfloat16, device="cuda")
    z = torch.empty((B, zd), dtype=torch.bfloat16, device="cuda")
    a = torch.empty((B, Hv), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((B, Hv), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_in_proj(s, I.HIDDEN, dev(P["x_norm"], "bf16"), dev(P["w_qkv"], "bf16"), dev(P["w_z"], "bf16"),
                    dev(P["w_a"], "bf16"), dev(P["w_b"], "bf16"), qkv, z, a, b)
    conv_state, state = dev(data["conv_state"], "bf16"), dev(data["state"], "f32")
    out = torch.empty((B, zd), dtype=torch.float32, device="cuda")
    gdn.gdn_decode_layer(s, conv_state, state, qkv, dev(data["conv_w"], "bf16"), a, b, z, dev(data["A_log"], "f32"),
                         dev(data["dt_bias"], "f32"), dev(data["norm_w"], "f32"), out)
    torch.cuda.synchronize()
    bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
    so = O.shape_of(cfg)
    cs = I.widen(data["conv_state"], "bf16").astype(np.float64)
    st = data["state"].astype(np.float64)
    ref = O.decode_step(so, cs, st, bf(bits(qkv)), I.widen(data["conv_w"], "bf16"), bf(bits(a)), bf(bits(b)),
                        bf(bits(z)), data["A_log"], data["dt_bias"], data["norm_w"])
    compare("in_proj -> decode_layer", host_f64(out), ref, "bf16", TOL["bf16"])


@pytest.mark.parametrize("B", [64, 100, 150, 300, 400])
def test_out_proj_deep_stages_ragged_columns(B):
    """out_proj's 4096-long contraction onto 1000 output columns, whose last column tile
    is ragged, through each 128-deep ring: 16 x 16 (B = 64 in the common stage order,
    100 in the staggered one, ragged rows), 32 x 16 (150 staggered, 300 common) and
    32 x 32 (400)."""
    hidden = 1000
    cfg = cfg_of(B)
    zd = cfg.z_dim
    rng = np.random.default_rng(B + 7)
    g = I.f32_to_bf16_bits(rng.standard_normal((B, zd), dtype=np.float32))
    w = I.f32_to_bf16_bits((rng.standard_normal((hidden, zd)) / np.sqrt(zd)).astype(np.float32))
    gd, wd = dev(g, "bf16"), dev(w, "bf16")
    y32 = torch.full((B, hidden), float("nan"), dtype=torch.float32, device="cuda")
    y16 = torch.full((B, hidden), float("nan"), dtype=torch.bfloat16, device="cuda")
    gdn.gdn_out_proj(shape_for(cfg), hidden, gd, wd, y32)
    gdn.gdn_out_proj(shape_for(cfg, out_dtype="bf16"), hidden, gd, wd, y16)
    torch.cuda.synchronize()
    idx = np.unique(np.array([0, 1, 31, 32, B // 2, B - 2, B - 1]))
    ref = O.linear(bf(g[idx]), bf(w))
    sel = torch.as_tensor(idx, device="cuda")
    check_f32("out_proj h1000 B=%d f32" % B, y32[sel], ref)
    check_bf16("out_proj h1000 B=%d bf16" % B, y16[sel], ref)
