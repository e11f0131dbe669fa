"""Pins of the oracle's MXFP8 (E4M3) storage encoding of compressed KV
entries (ai-papers.net article, hybrid attention section: most KV entries in
FP8; studioglobal.ai answer, FP4/FP8 mixed precision; OCP Microscaling v1.0
for the block format).

Independent references: torch's own float8_e4m3fn decode and round-to-
nearest-even conversion (a library routine, CPU), closed-form values of the
format, the scale rule at its boundaries, ties, saturation, and invariants
(idempotence, error bound)."""
import numpy as np
import pytest
import torch

import oracle


def block(values, fill=0.0):
    """One 32-value row holding `values` first."""
    row = np.full(32, fill, np.float64)
    row[:len(values)] = values
    return row[None, :]


def test_decode_matches_torch_for_every_code():
    codes = torch.arange(0, 127, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(127)])
    assert np.array_equal(got, ref)
    neg = (codes | 0x80).view(torch.float8_e4m3fn).double().numpy()
    got_neg = np.array([oracle.mxfp8_value(c | 0x80, 127) for c in range(127)])
    assert np.array_equal(got_neg, neg)


def test_closed_form_values():
    assert oracle.e4m3_value(0x01) == 2.0 ** -9          # smallest subnormal
    assert oracle.e4m3_value(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert oracle.e4m3_value(0x08) == 2.0 ** -6          # smallest normal
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x3C) == 1.5
    assert oracle.e4m3_value(0x7E) == 448.0              # largest finite
    assert oracle.mxfp8_value(0x38, 127 + 5) == 32.0
    assert oracle.mxfp8_value(0xB8, 127 - 3) == -0.125


def test_scale_rule_boundaries():
    # e = floor(log2 amax) - 8, stored as e + 127
    for amax, e in ((1.0, -8), (448.0, 0), (511.0, 0), (512.0, 1), (256.0, 0), (255.9, -1),
                    (2.0 ** 100, 92), (3.0 * 2.0 ** -120, -127)):
        _, s = oracle.quant_mxfp8(block([amax, -amax / 3]))
        assert s[0, 0] == e + 127, (amax, s[0, 0])
    c, s = oracle.quant_mxfp8(np.zeros((1, 32)))
    assert s[0, 0] == 0 and not c.any()


def test_saturation_and_signed_zero():
    c, s = oracle.quant_mxfp8(block([511.0, -470.0, 460.0, -0.0]))
    assert s[0, 0] == 127
    assert list(c[0, :4]) == [0x7E, 0xFE, 0x7E, 0x80]


def test_ties_go_to_the_even_code():
    # a block scaled by 2^0 (max 300)
    c, s = oracle.quant_mxfp8(block([300.0, 1.0625, 1.1875, 1.5 * 2 ** -9, 0.5 * 2 ** -9,
                                     2.5 * 2 ** -9, 17.0, 19.0]))
    assert s[0, 0] == 127
    # 1.0625: between 1 (0x38) and 1.125 (0x39) -> 0x38; 1.1875 -> 1.25 (0x3A);
    # 1.5 * 2^-9 -> code 2; 0.5 * 2^-9 -> 0; 2.5 * 2^-9 -> code 2;
    # 17 (16 and 18) -> 16 (0x58); 19 (18 and 20) -> 20 (0x5A)
    assert list(c[0, 1:8]) == [0x38, 0x3A, 0x02, 0x00, 0x02, 0x58, 0x5A]


def test_matches_torch_rounding_when_the_scale_is_one():
    rng = np.random.default_rng(11)
    x = rng.uniform(-463.0, 463.0, (64, 32))
    x[:, 0] = 300.0                                    # every block has e = 0
    x[:, 1:8] = rng.uniform(-2.0 ** -5, 2.0 ** -5, (64, 7))   # subnormal range
    c, s = oracle.quant_mxfp8(x)
    assert (s == 127).all()
    ref = torch.from_numpy(x).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(c, ref)


def test_scaled_blocks_match_torch_on_the_scaled_values():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((40, 128)) * np.exp2(rng.integers(-30, 30, (40, 1)))
    c, s = oracle.quant_mxfp8(x)
    e = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    y = np.ldexp(x, -e)                                # exact: powers of two
    y = np.clip(y, -448.0, 448.0)                      # saturation
    ref = torch.from_numpy(y).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(c, ref)


def test_round_trip_is_idempotent_and_within_half_a_step():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((50, 64)) * 3.0
    c, s = oracle.quant_mxfp8(x)
    dq = oracle.dequant_mxfp8(c, s)
    c2, s2 = oracle.quant_mxfp8(dq)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    # error: at most half a step of the value's binade (3 mantissa bits), or
    # half a subnormal step, unless saturated
    e = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    y = np.abs(np.ldexp(x, -e))
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(y, 1e-300))) - 3))
    bound = np.ldexp(step / 2, e)
    sat = y > 448.0
    assert (np.abs(dq - x)[~sat] <= bound[~sat]).all()


@pytest.mark.parametrize("d", [31, 0])
def test_rejects_bad_width(d):
    with pytest.raises(ValueError):
        oracle.quant_mxfp8(np.zeros((2, d)))
