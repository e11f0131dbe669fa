"""Pins of the oracle's softmax-gated pooling (jiwasawa.github.io post, CSA
token-level compression; studioglobal.ai answer, CSA bullet).

Each test checks the oracle against something other than its own formula:
closed forms (mean, identity, copy, two-point logistic), invariances and
the convex-hull property."""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(1234)


def test_uniform_gate_gives_block_mean():
    # equal logits inside a block -> equal weights 1/m -> arithmetic mean
    B, T, C, m = 2, 40, 8, 4
    x = RNG.standard_normal((B, T, C))
    per_block = RNG.standard_normal((B, T // m, C))
    gate = np.repeat(per_block, m, axis=1)
    out = oracle.compress(x, gate, m)
    ref = x.reshape(B, T // m, m, C).mean(axis=2)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-14)


def test_uniform_token_gate_gives_block_mean_m128():
    B, T, C, m = 1, 512, 4, 128
    x = RNG.standard_normal((B, T, C))
    gate = np.full((B, T, 1), 0.37)
    out = oracle.compress(x, gate, m)
    ref = x.reshape(B, T // m, m, C).mean(axis=2)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)


def test_m1_is_identity_bit_exact():
    x = RNG.standard_normal((2, 17, 8))
    gate = RNG.standard_normal((2, 17, 8)) * 5
    out = oracle.compress(x, gate, 1)
    assert np.array_equal(out, x)


def test_dominant_logit_copies_that_token_per_channel():
    # logit +200 at one token of each (block, channel): exp(-200) ~ 1e-87,
    # so the pooled value is that token's value of that channel
    B, T, C, m = 1, 32, 6, 4
    x = RNG.standard_normal((B, T, C))
    gate = np.zeros((B, T, C))
    pick = RNG.integers(0, m, size=(T // m, C))
    for j in range(T // m):
        for c in range(C):
            gate[0, m * j + pick[j, c], c] = 200.0
    out = oracle.compress(x, gate, m)
    ref = np.array([[x[0, m * j + pick[j, c], c] for c in range(C)] for j in range(T // m)])
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-80)


def test_two_token_logistic_closed_form():
    # softmax of two logits (a, b) is (sigmoid(a-b), sigmoid(b-a))
    B, T, C = 1, 20, 5
    x = RNG.standard_normal((B, T, C))
    z = RNG.standard_normal((B, T, C)) * 3
    out = oracle.compress(x, z, 2)
    a, b = z[0, 0::2], z[0, 1::2]
    ref = x[0, 0::2] / (1 + np.exp(b - a)) + x[0, 1::2] / (1 + np.exp(a - b))
    np.testing.assert_allclose(out[0], ref, rtol=1e-13, atol=1e-14)


def test_shift_invariance_per_block():
    B, T, C, m = 1, 64, 8, 8
    x = RNG.standard_normal((B, T, C))
    z = RNG.standard_normal((B, T, C))
    shift = np.repeat(RNG.standard_normal((B, T // m, C)) * 50, m, axis=1)
    np.testing.assert_allclose(oracle.compress(x, z + shift, m), oracle.compress(x, z, m),
                               rtol=1e-12, atol=1e-13)


def test_token_gate_equals_broadcast_channel_gate():
    B, T, C, m = 2, 24, 8, 4
    x = RNG.standard_normal((B, T, C))
    g = RNG.standard_normal((B, T, 1))
    a = oracle.compress(x, g, m)
    b = oracle.compress(x, np.repeat(g, C, axis=2), m)
    assert np.array_equal(a, b)


def test_partial_trailing_block_is_dropped():
    B, T, C, m = 1, 10, 4, 4
    x = RNG.standard_normal((B, T, C))
    z = RNG.standard_normal((B, T, C))
    out = oracle.compress(x, z, m)
    assert out.shape == (1, 2, C)
    np.testing.assert_array_equal(out, oracle.compress(x[:, :8], z[:, :8], m))


def test_convex_hull():
    B, T, C, m = 1, 128, 16, 16
    x = RNG.standard_normal((B, T, C))
    z = RNG.standard_normal((B, T, C)) * 4
    out = oracle.compress(x, z, m)
    blk = x.reshape(B, T // m, m, C)
    assert np.all(out <= blk.max(axis=2) + 1e-14)
    assert np.all(out >= blk.min(axis=2) - 1e-14)


@pytest.mark.parametrize("bad", [dict(m=0), dict(gc=3)])
def test_rejects_bad_arguments(bad):
    x = np.zeros((1, 8, 4))
    g = np.zeros((1, 8, bad.get("gc", 4)))
    with pytest.raises(ValueError):
        oracle.compress(x, g, bad.get("m", 4))
