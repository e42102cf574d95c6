"""Pins of the E4M3 oracle (oracle/lowp_gemm.py) against the format's definition and exact arithmetic."""
import numpy as np
import pytest

from oracle import lowp_gemm as lg


def test_decode_table_hand_values():
    d = lg.e4m3_decode_table()
    # values worked out from the definition: bias 7, 3 mantissa bits, subnormals m 2^-9
    assert d[0x00] == 0.0
    assert d[0x01] == 2.0 ** -9                # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9            # largest subnormal
    assert d[0x08] == 2.0 ** -6                # smallest normal
    assert d[0x38] == 1.0
    assert d[0x39] == 1.125
    assert d[0x40] == 2.0
    assert d[0x7E] == 448.0                    # largest finite
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert d[0xB8] == -1.0 and d[0x80] == 0.0
    finite = d[np.isfinite(d)]
    assert len(finite) == 254
    assert np.all(np.diff(d[:0x7F]) > 0)       # codes 0..0x7E increase with value
    assert np.all(d[0x80:0xFF] == -d[0x00:0x7F])


def test_encode_round_trips_every_finite_code():
    d = lg.e4m3_decode_table()
    codes = np.array([c for c in range(256) if np.isfinite(d[c]) and c != 0x80], dtype=np.uint8)
    assert np.array_equal(lg.e4m3_encode(d[codes]), codes)
    assert lg.e4m3_encode(np.array([-0.0]))[0] == 0


def test_encode_ties_go_to_the_even_code():
    # midpoint of 1.0 (0x38, even) and 1.125 (0x39): to 0x38; of 1.125 and 1.25 (0x3A, even): to 0x3A
    assert lg.e4m3_encode(np.array([1.0625]))[0] == 0x38
    assert lg.e4m3_encode(np.array([1.1875]))[0] == 0x3A
    # just above / below a midpoint
    assert lg.e4m3_encode(np.array([1.0625 + 1e-9]))[0] == 0x39
    assert lg.e4m3_encode(np.array([1.1875 - 1e-9]))[0] == 0x39
    # subnormal midpoint between 0 and 2^-9: to zero (even); above it: 2^-9
    assert lg.e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00
    assert lg.e4m3_encode(np.array([1.5 * 2.0 ** -10]))[0] == 0x01
    # midpoint between the largest subnormal 7 2^-9 (0x07, odd) and 2^-6 (0x08, even): to 0x08
    assert lg.e4m3_encode(np.array([7.5 * 2.0 ** -9]))[0] == 0x08
    # saturation
    assert lg.e4m3_encode(np.array([449.0, 1e9, -1e9]))[0] == 0x7E
    assert lg.e4m3_encode(np.array([-1e9]))[0] == 0xFE


def test_encode_is_the_nearest_value_by_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000) * 10 ** rng.uniform(-4, 2.5, 4000), rng.uniform(-448, 448, 2000)])
    codes = lg.e4m3_encode(x)
    d = lg.e4m3_decode_table()
    finite = np.array([c for c in range(256) if np.isfinite(d[c])])
    dist = np.abs(x[:, None] - d[finite][None, :])
    best = dist.min(axis=1)
    got = np.abs(x - d[codes.astype(np.int64)])
    assert np.all(got == best)


def test_quantize_rows_maps_the_row_maximum_to_448():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 37)).astype(np.float32)
    x[3] = 0.0
    codes, s = lg.quantize_rows(x)
    d = lg.e4m3_decode(codes)
    for i in (0, 1, 2, 4):
        j = np.argmax(np.abs(x[i]))
        assert abs(d[i, j]) == 448.0
        assert s[i] == np.float32(np.abs(x[i]).max()) / np.float32(448)
    assert s[3] == 0 and np.all(codes[3] == 0)
    # the dequantised values are within half an E4M3 spacing (relative 2^-4) of x, plus subnormal slack
    err = np.abs(d * s[:, None] - x)
    assert np.all(err <= np.abs(x) * 2.0 ** -4 + s[:, None] * 2.0 ** -10)


def test_gemm_is_exact_integer_arithmetic_on_integer_codes():
    # codes whose values are the integers 1..16 (exact in E4M3) and their negatives
    d = lg.e4m3_decode_table()
    ints = {int(v): c for c, v in enumerate(d) if np.isfinite(v) and v == int(v) and 1 <= v <= 16}
    keys = sorted(ints)
    rng = np.random.default_rng(5)
    ai = rng.choice(keys, size=(7, 300)) * rng.choice([-1, 1], size=(7, 300))
    wi = rng.choice(keys, size=(9, 300)) * rng.choice([-1, 1], size=(9, 300))
    enc = lambda m: np.vectorize(lambda v: ints[abs(v)] | (0x80 if v < 0 else 0))(m).astype(np.uint8)
    sa = np.full(7, 0.5)
    sw = np.full(9, 0.25)
    c = lg.gemm_e4m3(enc(ai), sa, enc(wi), sw)
    exact = (ai.astype(np.int64) @ wi.T.astype(np.int64)).astype(np.float64) * 0.125
    assert np.array_equal(c, exact)


def test_bf16_round_ties_to_even():
    assert lg.bf16_round(np.array([1.0]))[0] == 1.0
    assert lg.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0                   # tie -> even
    assert lg.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6   # tie -> even (up)
    assert lg.bf16_round(np.array([1.0 + 2.0 ** -8 + 2.0 ** -12]))[0] == 1.0 + 2.0 ** -7
