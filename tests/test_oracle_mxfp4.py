"""Pins of the oracle's MXFP4 encoder (studioglobal.ai answer, FP4/FP8 mixed
precision section: MXFP4, two values per byte; e2m1 elements with one
power-of-two scale per 32 values).

Checks against the e2m1 bit-field definition, a hand-derived table of tie
and saturation points (tests/golden/mxfp4_rounding.json), brute-force
nearest-value search, the scale-exponent property and idempotence."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_rounding.json")
RNG = np.random.default_rng(7)


def e2m1_from_bits(code: int) -> float:
    """e2m1 by its bit fields: sign | 2-bit exponent (bias 1) | 1-bit mantissa;
    exponent field 0 is subnormal (0.5 * mantissa)."""
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    mant = code & 1
    if e == 0:
        return s * 0.5 * mant
    return s * 2.0 ** (e - 1) * (1 + mant / 2)


def decode(codes, scales, d):
    """Dequantise rows (independent of the oracle's own table)."""
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    out = np.zeros(codes.shape[:-1] + (d,))
    for idx in np.ndindex(codes.shape[:-1]):
        for i in range(d):
            byte = int(codes[idx + (i // 2,)])
            c = byte & 0xF if i % 2 == 0 else byte >> 4
            out[idx + (i,)] = e2m1_from_bits(c) * 2.0 ** (int(scales[idx + (i // 32,)]) - 127)
    return out


def test_value_table_matches_bit_fields_exhaustively():
    for code in range(16):
        for scale in range(0, 255):
            assert oracle.mxfp4_value(code, scale) == e2m1_from_bits(code) * 2.0 ** (scale - 127)


def test_tie_and_saturation_table():
    cases = json.load(open(GOLDEN))["cases"]
    for x, want in cases:
        blk = np.zeros(32)
        blk[0] = x
        blk[5] = 6.0        # forces the block exponent e = 0
        codes, scales = oracle.quant_mxfp4(blk[None, :])
        assert scales[0, 0] == 127, x
        assert codes[0, 0] & 0xF == want, (x, codes[0, 0] & 0xF, want)


def test_scale_exponent_rule():
    # nonzero, unclamped block: max|x| * 2^-e lies in [4, 8)
    x = RNG.standard_normal((200, 64)) * np.exp(RNG.uniform(-20, 20, size=(200, 1)))
    codes, scales = oracle.quant_mxfp4(x)
    for r in range(200):
        for b in range(2):
            amax = np.abs(x[r, 32 * b:32 * b + 32]).max()
            e = int(scales[r, b]) - 127
            assert 4.0 <= amax * 2.0 ** (-e) < 8.0


def test_zero_block():
    codes, scales = oracle.quant_mxfp4(np.zeros((1, 32)))
    assert scales[0, 0] == 0 and not codes.any()


def test_nearest_by_brute_force_with_ties_to_even():
    x = RNG.standard_normal((64, 32))
    # sprinkle exact tie points of the block's grid
    codes, scales = oracle.quant_mxfp4(x)
    got = decode(codes, scales, 32)
    for r in range(64):
        sc = 2.0 ** (int(scales[r, 0]) - 127)
        grid = np.array([e2m1_from_bits(c) * sc for c in range(16)])
        for i in range(32):
            v = x[r, i]
            dist = np.abs(grid - v)
            best = dist.min()
            if abs(v) > 6 * sc:                      # saturation
                assert got[r, i] == np.sign(v) * 6 * sc
                continue
            assert abs(got[r, i] - v) == best
            byte = int(codes[r, i // 2])
            c = byte & 0xF if i % 2 == 0 else byte >> 4
            ties = [k for k in range(8) if dist[k if v >= 0 else k + 8] == best]
            if len(ties) > 1:                       # tie -> even code
                assert (c & 7) % 2 == 0


def test_grid_values_round_trip_exactly():
    s = RNG.integers(-30, 30, size=(50, 1))
    mags = np.array([e2m1_from_bits(c) for c in range(8)])
    vals = RNG.choice(mags, size=(50, 32)) * RNG.choice([-1, 1], size=(50, 32))
    vals[:, 0] = 6.0
    x = vals * 2.0 ** s
    codes, scales = oracle.quant_mxfp4(x)
    assert np.array_equal(decode(codes, scales, 32), x)


def test_idempotent():
    x = RNG.standard_normal((40, 64)) * 3
    c1, s1 = oracle.quant_mxfp4(x)
    c2, s2 = oracle.quant_mxfp4(decode(c1, s1, 64))
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("pos", [0, 1, 30, 31, 32, 63])
def test_nibble_order(pos):
    x = np.zeros((1, 64))
    x[0, pos] = 1.0
    codes, scales = oracle.quant_mxfp4(x)
    byte = codes[0, pos // 2]
    want = 6           # 1.0 with e = -2 is 4.0 -> code 6
    assert (byte & 0xF if pos % 2 == 0 else byte >> 4) == want
    assert int(codes.astype(np.int64).sum()) == (want if pos % 2 == 0 else want << 4)


def test_negative_zero_keeps_sign_bit():
    x = np.zeros((1, 32))
    x[0, 0] = -0.0
    x[0, 1] = -0.01
    x[0, 2] = 6.0
    codes, _ = oracle.quant_mxfp4(x)
    assert codes[0, 0] == 0x88
