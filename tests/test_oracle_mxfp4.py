"""Pins of the oracle's MXFP4 weight codec (the W4A8 workload) against the
OCP Microscaling (MX) formats definition: the E2M1 element values, the E8M0
scale values, the packing order, and the error bound of the generator's MX
conversion as the oracle decodes it."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle


def test_e2m1_values_from_the_format_definition():
    # E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
    # subnormal. The eight magnitudes the MX definition lists:
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = oracle.e2m1_to_f64(np.arange(16))
    np.testing.assert_array_equal(got[:8], mags)
    np.testing.assert_array_equal(got[8:], [-m for m in mags])
    assert np.signbit(got[8])                      # code 8 is -0


def test_e8m0_values():
    got = oracle.e8m0_to_f64(np.array([0, 1, 126, 127, 128, 130, 254, 255]))
    np.testing.assert_array_equal(got[:7], [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 8.0, 2.0 ** 127])
    assert np.isnan(got[7])


def test_packing_order_and_block_scales():
    # one row of 64 elements: byte 0 = 0x21 holds element 0 = code 1 (0.5) in
    # its low nibble and element 1 = code 2 (1.0) in its high nibble; byte 31
    # = 0xF7 holds code 7 (6.0) and code 15 (-6.0); block 1 has scale 2^3
    packed = np.zeros((1, 32), np.uint8)
    packed[0, 0] = 0x21
    packed[0, 31] = 0xF7
    scales = np.array([[127, 130]], np.uint8)
    w = oracle.decode_mxfp4(packed, scales)
    assert w.shape == (1, 64)
    assert w[0, 0] == 0.5 and w[0, 1] == 1.0
    assert w[0, 62] == 6.0 * 8 and w[0, 63] == -6.0 * 8
    assert np.count_nonzero(w) == 4
    # a plausible slip, the nibbles swapped, gives another matrix
    swapped = ((packed & 0xF) << 4) | (packed >> 4)
    assert not np.array_equal(oracle.decode_mxfp4(swapped, scales), w)


def _e2m1_bound(y):
    """Largest rounding error of |y| on the E2M1 grid, saturating at 6."""
    return np.where(y <= 2.0, 0.25, np.where(y <= 4.0, 0.5, np.where(y <= 6.0, 1.0, y - 6.0)))


@pytest.mark.parametrize("shape", [(64, 128), (7, 2048)])
def test_generator_conversion_within_the_mx_bound(shape):
    """The generator's MX conversion, decoded by the oracle: every element is
    within half a grid step of its source, and the shared exponent puts the
    block's largest magnitude on the top exponent of E2M1 (4 or 6)."""
    g = torch.Generator().manual_seed(3)
    x = torch.randn(shape, generator=g) * 0.02
    x[0, :32] = 0.0                                 # an all-zero block
    packed, scales = moe_synth._quant_mxfp4_rows(x)
    deq = oracle.decode_mxfp4(packed.numpy(), scales.numpy())
    v = x.double().numpy()
    X = np.repeat(oracle.e8m0_to_f64(scales.numpy()), 32, axis=1)
    y = np.abs(v) / X
    assert np.all(np.abs(deq - v) <= _e2m1_bound(y) * X * (1 + 1e-12))
    assert np.all(deq[0, :32] == 0.0)
    blk = np.abs(deq.reshape(shape[0], -1, 32) / X.reshape(shape[0], -1, 32)).max(axis=2)
    nz = np.abs(v.reshape(shape[0], -1, 32)).max(axis=2) > 0
    assert np.all(np.isin(blk[nz], [4.0, 6.0]))


def test_w4a8_layer_equals_dense_bruteforce():
    cfg = moe_synth.make_config("tiny", dtype="w4a8_mxfp4", T=128, num_segments=8, E_global=8, k=2,
                                e_begin=1, e_end=6)
    inp = moe_synth.generate(cfg)
    r = oracle.moe_layer(inp, cfg)
    yb = oracle.moe_layer_bruteforce(inp, cfg)
    q = oracle.y_row_of_token(np.arange(cfg.T), cfg.T, cfg.num_segments)
    np.testing.assert_allclose(r["Y"][q], yb, rtol=1e-11, atol=1e-15)
    assert np.abs(r["Y"]).max() > 0
