"""Pins of the oracle's number formats against their definitions and against
library casts (torch's fp32 -> bfloat16 and fp32 -> float8_e4m3fn conversions
both round to nearest even)."""
import numpy as np
import pytest
import torch

import oracle



@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
    (1.0 + 2.0 ** -8, 0x3F80),          # tie between mantissa 0 and 1 -> even (0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),      # tie between mantissa 1 and 2 -> even (2)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),   # just above the tie -> up
    (3.0e38, 0x7F62), (3.5e38, 0x7F80),       # 3.5e38 is above the bf16 max (~3.39e38): inf
    (2.0 ** -133, 0x0001),              # smallest subnormal
    (2.0 ** -134, 0x0000),              # half of it: tie -> even (zero)
])
def test_bf16_worked_values(x, bits):
    assert int(oracle.f64_to_bf16_bits(np.float64(x))) == bits
    if bits != 0x7F80:
        assert oracle.bf16_bits_to_f64(np.uint16(bits)) == oracle.round_to_bf16(x)


def test_bf16_matches_torch_cast_on_fp32():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-30, 1e-3, 1.0, 1e20)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(x.astype(np.float64)), ref)


def test_bf16_round_is_nearest_representable():
    """Direct from the definition: the result is representable, and no other
    bf16 value is closer (checked via the two neighbouring bf16 codes)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(50000) * 3.0
    r = oracle.round_to_bf16(x)
    bits = oracle.f64_to_bf16_bits(x).astype(np.int64)
    assert np.all(oracle.bf16_bits_to_f64(bits.astype(np.uint16)) == r)
    for nb in (bits - 1, bits + 1):
        other = oracle.bf16_bits_to_f64((nb & 0xFFFF).astype(np.uint16))
        assert np.all(np.abs(x - r) <= np.abs(x - other))


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x38), (-1.0, 0xB8), (448.0, 0x7E), (-448.0, 0xFE),
    (1000.0, 0x7E),                     # saturates
    (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07), (2.0 ** -6, 0x08),
    (2.0 ** -10, 0x00),                 # tie between 0 and 2^-9 -> even (0)
    (3 * 2.0 ** -10, 0x02),             # tie between 1 and 2 (x 2^-9) -> even (2)
    (1.0625, 0x38), (1.1875, 0x3A),     # ties at 1.0 + 1/16, 1.125 + 1/16
    (240.0, 0x77), (256.0, 0x78), (0.0, 0x00),
])
def test_e4m3_worked_values(x, bits):
    assert int(oracle.f64_to_e4m3_bits(np.float64(x))) == bits


def test_e4m3_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = oracle.e4m3_bits_to_f64(codes)
    same = (ref == got) | (np.isnan(ref) & np.isnan(got))
    assert same.all()
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0


def test_e4m3_encode_matches_torch_cast_within_range():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(100000) * s for s in (0.01, 1.0, 100.0)]).astype(np.float32)
    x = np.clip(x, -448.0, 448.0)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.f64_to_e4m3_bits(x.astype(np.float64)), ref)


def test_row_quantiser_properties():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((6, 384)) * np.array([1e-3, 1.0, 30.0, 0.0, 5.0, 2.0])[:, None]
    a[4, 128:256] = 0.0
    codes, scale, deq = oracle.quantize_rows_e4m3(a, 128)
    assert scale.dtype == np.float32 and scale.shape == (6, 3)
    assert np.all(scale[3] == 1.0) and scale[4, 1] == 1.0       # all-zero blocks keep scale 1
    assert np.all(deq[3] == 0.0)
    blocks = np.abs(a).reshape(6, 3, 128)
    amax = blocks.max(axis=2)
    nz = amax > 0
    # the block's largest element maps to (within rounding) the top code 448
    top = np.abs(oracle.e4m3_bits_to_f64(codes.reshape(6, 3, 128))).max(axis=2)
    assert np.all(top[nz] == 448.0)
    # relative error of every element is bounded by half an e4m3 ulp of its block's grid
    err = np.abs(deq - a).reshape(6, 3, 128)
    bound = np.maximum(blocks * 2.0 ** -4, 2.0 ** -10 * scale[:, :, None]) * (1 + 1e-6)
    assert np.all(err <= bound + 1e-300)
