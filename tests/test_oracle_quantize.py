"""Pins of the oracle's NVFP4 quantiser (an encoding, so pinned by brute
force, closed-form bounds and invariants rather than by a second copy)."""
import numpy as np
import pytest

from oracle import nvfp4_oracle as O

E2M1_MAG = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _brute_e4m3(v):
    """Nearest finite non-negative E4M3 code by exhaustive search; ties to
    the even code; saturating."""
    vals = np.array([O.decode_e4m3(c) for c in range(0x7F)])
    d = np.abs(vals - v)
    best = np.flatnonzero(d == d.min())
    if len(best) == 2:
        return int(best[0] if best[0] % 2 == 0 else best[1])
    return int(best[0])


def _brute_e2m1(v):
    d = np.abs(E2M1_MAG - abs(v))
    best = np.flatnonzero(d == d.min())
    c = int(best[0] if len(best) == 1 or best[0] % 2 == 0 else best[1])
    return c | (8 if np.signbit(v) else 0)


def test_e4m3_rounding_brute_force():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        np.exp2(rng.uniform(-12, 10, 4000)),
        rng.uniform(0, 2.0 ** -6, 500),        # subnormal range
        np.array([0.0, 448.0, 449.0, 464.0, 1e6, 2.0 ** -10, 3 * 2.0 ** -11]),
    ]).astype(np.float32)
    got = O.e4m3_rne_saturate(v)
    for x, c in zip(v, got):
        assert c == _brute_e4m3(float(x)), (x, c)


def test_e4m3_midpoints_go_to_even():
    vals = O.decode_e4m3(np.arange(0x7F))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    got = O.e4m3_rne_saturate(mids).astype(int)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, expect)


def test_e2m1_rounding_ties_listed():
    # half-way points and where they must go (even mantissa)
    cases = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             0.2499: 0, 0.2501: 1, 5.0001: 7, 7.0: 7, 100.0: 7, 0.0: 0}
    for v, c in cases.items():
        assert O.e2m1_rne_saturate(v) == c, v
        assert O.e2m1_rne_saturate(-v) == c | 8, -v


def test_e2m1_rounding_brute_force():
    rng = np.random.default_rng(3)
    v = rng.uniform(-8, 8, 5000).astype(np.float32)
    got = O.e2m1_rne_saturate(v)
    for x, c in zip(v, got):
        assert c == _brute_e2m1(float(x))


def _rand_matrix(rng, n, k, scale=1.0):
    return (rng.standard_normal((n, k)) * scale).astype(np.float32)


def test_quantize_codes_are_nearest_for_the_chosen_scale():
    rng = np.random.default_rng(7)
    x = _rand_matrix(rng, 8, 64, 0.02)
    codes, scales, g = O.quantize(x)
    el = O.unpack_nibbles(codes)
    s_dec = O.decode_e4m3(scales).astype(np.float32)
    for r in range(8):
        for b in range(4):
            denom = np.float32(s_dec[r, b] * g)
            inv = np.float32(np.float32(1) / denom)
            for i in range(16):
                v = np.float32(x[r, 16 * b + i] * inv)
                assert el[r, 16 * b + i] == _brute_e2m1(float(v))


def test_quantize_error_bound():
    # |x - deq| <= half the local E2M1 spacing times s*g, plus fp32 slack
    rng = np.random.default_rng(11)
    x = _rand_matrix(rng, 32, 256, 0.02)
    codes, scales, g = O.quantize(x)
    deq = O.dequantize(codes, scales, g)
    s = np.repeat(O.decode_e4m3(scales), 16, axis=1) * np.float64(g)
    mag = np.abs(deq) / np.where(s > 0, s, 1)
    spacing = np.where(mag < 2, 0.5, np.where(mag < 4, 1.0, 2.0))
    # element not saturated: |x|/(s g) <= 6
    unsat = np.abs(x) <= 6 * s * (1 + 1e-6)
    err = np.abs(x.astype(np.float64) - deq)
    bound = 0.5 * spacing * s * (1 + 1e-6) + 1e-30
    assert np.all(err[unsat] <= bound[unsat])


def test_tensor_amax_block_gets_max_scale():
    rng = np.random.default_rng(13)
    for _ in range(20):
        x = _rand_matrix(rng, 4, 128, float(np.exp(rng.uniform(-10, 10))))
        codes, scales, g = O.quantize(x)
        assert g == np.float32(np.abs(x).max() / np.float32(2688.0))
        r, c = np.unravel_index(np.argmax(np.abs(x)), x.shape)
        assert scales[r, c // 16] == 0x7E
        # the amax element itself maps to +-6
        assert O.unpack_nibbles(codes)[r, c] & 7 == 7


def test_round_trip_normal_blocks():
    rng = np.random.default_rng(17)
    x = _rand_matrix(rng, 16, 256, 0.02)
    codes, scales, g = O.quantize(x)
    deq = O.dequantize_f32(codes, scales, g)
    c2, s2, g2 = O.quantize(deq, g=g)
    normal = scales >= 0x08
    assert normal.mean() > 0.9
    assert np.array_equal(s2[normal], scales[normal])
    el1 = O.unpack_nibbles(codes).reshape(16, 16, 16)
    el2 = O.unpack_nibbles(c2).reshape(16, 16, 16)
    # identical codes up to the sign of zero (a dequantised -0 code is +0)
    same = (el1 == el2) | ((el1 & 7) == 0) & ((el2 & 7) == 0)
    assert np.all(same[normal])
    # every block's largest code is 6
    assert np.all((el1 & 7).max(axis=2)[normal] == 7)


def test_sign_symmetry():
    rng = np.random.default_rng(19)
    x = _rand_matrix(rng, 8, 128)
    c1, s1, g1 = O.quantize(x)
    c2, s2, g2 = O.quantize(-x)
    assert g1 == g2 and np.array_equal(s1, s2)
    assert np.array_equal(c2, c1 ^ 0x88)


@pytest.mark.parametrize("j", [-20, -3, 1, 7, 30])
def test_power_of_two_equivariance(j):
    rng = np.random.default_rng(23)
    x = _rand_matrix(rng, 8, 64)
    c1, s1, g1 = O.quantize(x)
    c2, s2, g2 = O.quantize((x * np.float32(2.0 ** j)).astype(np.float32))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert g2 == np.float32(g1 * np.float32(2.0 ** j))


def test_zero_tensor_and_zero_block():
    codes, scales, g = O.quantize(np.zeros((2, 32), np.float32))
    assert g == 1.0 and not codes.any() and not scales.any()
    x = np.zeros((1, 32), np.float32)
    x[0, 16:] = np.linspace(-1, 1, 16)
    codes, scales, g = O.quantize(x)
    assert scales[0, 0] == 0 and np.all(O.unpack_nibbles(codes)[0, :16] == 0)
    assert scales[0, 1] == 0x7E


def test_tiny_block_scale_underflows_to_zero_codes():
    # a block whose scale rounds to E4M3 zero gets +0 codes everywhere
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0
    x[0, 16] = -1e-7
    codes, scales, g = O.quantize(x)
    assert scales[0, 1] == 0
    assert np.all(O.unpack_nibbles(codes)[0, 16:] == 0)


def test_hand_worked_block():
    # g given as 1/64 (a power of two) and a block whose amax is 3.0:
    # s = 3 / (6/64) = 32 = 2^5 -> E4M3 exponent field 12, code 0x60; denom = 0.5; x/0.5 on the grid.
    g = np.float32(1.0 / 64)
    x = np.array([[3.0, -0.25, 0.125, 0.3, 0.75, -1.0, 1.5, 2.0,
                   0.0, -0.0, 1.25, 0.625, 2.9, -3.0, 0.1, 0.5]], np.float32)
    codes, scales, g2 = O.quantize(x, g=g)
    assert g2 == g and scales[0, 0] == 0x60 and O.decode_e4m3(0x60) == 32.0
    el = O.unpack_nibbles(codes)[0]
    # x / 0.5 = 6, -0.5, 0.25, 0.6, 1.5, -2, 3, 4, 0, -0, 2.5, 1.25, 5.8, -6, 0.2, 1
    expect = [7, 9, 0, 1, 3, 12, 5, 6, 0, 8, 4, 2, 7, 15, 0, 2]
    assert list(el) == expect


def test_quantize_rejects_bad_input():
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 24), np.float32))
    with pytest.raises(ValueError):
        O.quantize(np.full((1, 16), np.inf, np.float32))
