"""Pins of the oracle's element decoders, packing and bf16 rounding."""
import os

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_pairs(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            a, b = line.split()
            rows.append((int(a, 0), float(b)))
    return rows


def test_e2m1_table_exhaustive():
    rows = _read_pairs("e2m1_values.txt")
    assert [c for c, _ in rows] == list(range(16))
    got = O.decode_e2m1(np.arange(16))
    for code, value in rows:
        assert got[code] == value
        assert np.signbit(got[code]) == np.signbit(value), code


def test_e4m3_fixed_points():
    for code, value in _read_pairs("e4m3_points.txt"):
        got = O.decode_e4m3(code)
        if np.isnan(value):
            assert np.isnan(got), hex(code)
        else:
            assert got == value and np.signbit(got) == np.signbit(value), hex(code)


def test_e4m3_positive_codes_strictly_monotone_and_finite():
    v = O.decode_e4m3(np.arange(0x7F))
    assert np.all(np.isfinite(v))
    assert np.all(np.diff(v) > 0)
    assert v[-1] == 448.0 and len(np.unique(v)) == 127
    # negative half mirrors the positive half
    assert np.array_equal(O.decode_e4m3(np.arange(0x80, 0xFF)), -v)


def test_e4m3_matches_torch_float8():
    # independent library decoder of the same OCP type
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    ref = b.to(torch.float64).numpy()
    got = O.decode_e4m3(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_pack_unpack_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    codes = O.unpack_nibbles(b[None, :])[0]
    assert np.array_equal(codes[0::2], b & 15)
    assert np.array_equal(codes[1::2], b >> 4)
    assert np.array_equal(O.pack_nibbles(codes[None, :])[0], b)
    # element 2i is the low nibble: byte 0x21 holds codes (1, 2)
    assert list(O.unpack_nibbles(np.array([[0x21]], np.uint8))[0]) == [1, 2]


def test_block_values_products_exact_in_bf16_and_f16():
    # every e2m1 * e4m3 product is representable in bf16 and in fp16
    e = O.decode_e2m1(np.arange(16))
    s = O.decode_e4m3(np.arange(0x7F))
    prod = np.outer(e, s).ravel()
    assert np.array_equal(O.bf16_rne(prod), prod)
    assert np.array_equal(prod.astype(np.float16).astype(np.float64), prod)
    nz = np.abs(prod[prod != 0])
    assert nz.min() == 2.0 ** -10 and nz.max() == 2688.0


def test_bf16_rne_ties_and_torch():
    one = 1.0
    assert O.bf16_rne(one + 2.0 ** -8) == 1.0                     # tie -> even
    assert O.bf16_rne(one + 3 * 2.0 ** -8) == one + 2.0 ** -6    # tie -> even
    assert O.bf16_rne(one + 2.0 ** -8 + 2.0 ** -30) == one + 2.0 ** -7
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 1e-39).astype(np.float32),
                        (rng.standard_normal(2000) * 1e30).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_rne(x.astype(np.float64)), ref)


def test_dequantize_f32_is_single_rounding():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(4, 32), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(4, 4), dtype=np.uint8)
    g = np.float32(0.0123)
    d64 = O.dequantize(codes, scales, g)
    d32 = O.dequantize_f32(codes, scales, g)
    assert np.array_equal(d32, d64.astype(np.float32))
    # e2m1*e4m3 exact, so the fp32 product with g is the correctly rounded one
    bv = O.block_values(codes, scales).astype(np.float32)
    assert np.array_equal(d32, (bv * g).astype(np.float32))


@pytest.mark.parametrize("bad", [16, -1])
def test_decoders_reject_out_of_range(bad):
    with pytest.raises(ValueError):
        O.decode_e2m1(bad)
