"""Pins of the oracle's MX (microscaling) codecs and of the MXFP4 layer path:
the OCP MX v1.0 element and scale definitions, torch's own float8 casts, the
MX scale rule on worked values, and an exact special case of the layer."""
import numpy as np
import torch

import workloads as W
from oracle import e4m3
from oracle import moe as O
from oracle import mx


def test_e2m1_table_is_the_ocp_value_set():
    # OCP MX v1.0, FP4 E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = mx.e2m1_decode(np.arange(16))
    assert got[:8].tolist() == mags
    assert got[8:].tolist() == [-m for m in mags]
    assert np.signbit(got[8])          # code 8 is -0


def test_e8m0_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = mx.e8m0_decode(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_fp4_packing_order_and_dequant():
    packed = np.array([[0x21, 0xF7]], dtype=np.uint8)     # codes 1, 2, 7, 15
    assert mx.unpack_fp4(packed).tolist() == [[1, 2, 7, 15]]
    k = np.zeros((1, 16), dtype=np.uint8)
    k[0, 0] = 0x21                                       # elements 0, 1 = 0.5, 1.0
    w = mx.dequant_mxfp4(k, np.array([[128]], dtype=np.uint8))   # scale 2
    assert w[0, :4].tolist() == [1.0, 2.0, 0.0, 0.0] and w.shape == (1, 32)


def test_mxfp8_scale_rule_worked_values():
    def block(amax):
        v = np.zeros((1, 32), dtype=np.float32)
        v[0, 5] = amax
        return mx.quantise_mxfp8(v)
    # shared exponent = floor(log2(amax)) - 8, code = exponent + 127
    for amax, code in ((1.0, 119), (448.0, 127), (0.75, 118), (2.0 ** -20, 127 - 28), (3.0e38, 127 + 119)):
        assert block(amax)[1][0, 0] == code, amax
    # 511 sits above 448 * 2^0: its element saturates to the largest finite e4m3 code.
    c, s = block(511.0)
    assert s[0, 0] == 127 and e4m3.decode(c[0, 5]) == 448.0
    # An all-zero block: scale 2^0, zero codes.
    c, s = mx.quantise_mxfp8(np.zeros((2, 64), dtype=np.float32))
    assert (s == 127).all() and (c == 0).all()
    # Scales below 2^-127 clamp there.
    assert block(2.0 ** -126)[1][0, 0] == 0


def test_mxfp8_codes_match_torch_e4m3_cast():
    rng = np.random.default_rng(21)
    v = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-12, 12, size=(64, 1)))).astype(np.float32)
    codes, scales = mx.quantise_mxfp8(v)
    scaled = v.astype(np.float64) / np.repeat(mx.e8m0_decode(scales), 32, axis=1)
    ref = torch.from_numpy(np.clip(scaled, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(codes, ref.view(torch.uint8).numpy())


def test_mxfp8_error_bound_and_exact_round_trip():
    rng = np.random.default_rng(22)
    v = rng.standard_normal((32, 512)).astype(np.float32)
    q = mx.dequant_mxfp8(*mx.quantise_mxfp8(v))
    # Elements at least 1/64 of the block maximum are normal e4m3 after scaling:
    # relative error <= 2^-4 (3 mantissa bits, round to nearest) -- except where the
    # MX rule's scale leaves the element above 448 (a block maximum in [448, 512)
    # x 2^s), which saturates to 448 x 2^s: error below 1/8.
    amax = np.repeat(np.abs(v).reshape(32, -1, 32).max(axis=2), 32, axis=1)
    scale = np.repeat(mx.e8m0_decode(mx.quantise_mxfp8(v)[1]), 32, axis=1)
    big = np.abs(v) >= amax / 64
    sat = np.abs(v) / scale > 448
    ok = big & ~sat
    assert (np.abs(q - v)[ok] <= 2.0 ** -4 * np.abs(v)[ok]).all()
    assert sat.any() and (np.abs(q[sat]) == 448 * scale[sat]).all()
    assert (np.abs(q - v)[sat] < np.abs(v)[sat] / 8).all()
    # Values that are e4m3 numbers times the block scale survive exactly.
    codes = rng.integers(0, 0x7F, size=(8, 64)).astype(np.uint8)
    exact = (e4m3.decode(codes) * 2.0 ** -3).astype(np.float32)
    exact[:, ::32] = 448.0 * 2.0 ** -3          # pin each block's maximum so its scale is 2^-3
    q2 = mx.dequant_mxfp8(*mx.quantise_mxfp8(exact))
    assert np.array_equal(q2, exact.astype(np.float64))


def test_mxfp4_layer_with_mx_exact_inputs_is_the_plain_ffn():
    # With activations that MXFP8 represents exactly, the oracle's MXFP4 expert is
    # the float64 SwiGLU of the dequantised weights: x enters unchanged, and so does
    # h whenever h is exact too -- checked here on the gate/up half via a one-row
    # down projection of zeros except one MX-exact column.
    shape = W.DRAFTER.with_(name="t", hidden_size=128, moe_intermediate_size=64, n_routed_experts=2,
                            shared_expert_intermediate_size=0, weight_dtype=W.DT_MXFP4)
    w = W.expert_weights(shape, 5, 0)
    rng = np.random.default_rng(23)
    codes = rng.integers(0, 0x7F, size=(4, 128)).astype(np.uint8)
    x = (e4m3.decode(codes) * np.where(rng.random((4, 128)) < 0.5, -1, 1) * 2.0 ** -6).astype(np.float32)
    x[:, ::32] = 448.0 * 2.0 ** -6
    wg = mx.dequant_mxfp4(w["gate"].numpy(), w["gate_s"].numpy())
    wu = mx.dequant_mxfp4(w["up"].numpy(), w["up_s"].numpy())
    a = torch.from_numpy(x.astype(np.float64)) @ torch.from_numpy(wg).T
    b = torch.from_numpy(x.astype(np.float64)) @ torch.from_numpy(wu).T
    h_ref = (a * torch.sigmoid(a) * b).numpy()
    wd = mx.dequant_mxfp4(w["down"].numpy(), w["down_s"].numpy())
    y_ref = O._mx_activation(h_ref.astype(np.float32)) @ wd.T
    y = O.swiglu_ffn(x.astype(np.float64), w, W.DT_MXFP4)
    assert np.allclose(y, y_ref, rtol=1e-12, atol=1e-15)
