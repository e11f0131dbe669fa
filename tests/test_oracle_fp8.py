"""Pins of the oracle's FP8 attention arithmetic (reading R13d; ai-papers.net
article, hybrid attention section: most KV entries in FP8).

* quant_fp8_rows: E4M3 with one scale exponent per row.  Pinned to torch's
  float8_e4m3fn round-to-nearest-even conversion of the row scaled by its
  exponent (a library routine, CPU), to the exponent rule at its boundaries,
  and to the already pinned 32-value MXFP8 encoding on rows whose runs
  share one exponent.
* attend_stats: the weighted means amean = sum p|v| / sum p and
  rms = sqrt(sum p^2 v^2) / sum p, pinned to softmax weights from torch
  (CPU, fp64) and to closed forms (one key, equal scores).
* attend_fp8: the composition of the pinned pieces (queries encoded per
  head row, every row decoded exactly, exact attention)."""
import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(41)


def torch_e4m3(y):
    """Codes of torch's RNE conversion of y (|y| <= 448 after clipping)."""
    y = np.clip(y, -448.0, 448.0)
    return torch.from_numpy(y).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_rows_match_torch_rounding_at_the_row_exponent():
    x = RNG.standard_normal((60, 128)) * np.exp2(RNG.integers(-40, 40, (60, 1)))
    x[:5, 7:40] *= 1e-4                      # runs far below the row maximum
    c, s = oracle.quant_fp8_rows(x)
    assert (s == s[:, :1]).all()             # one exponent per row, repeated
    e = s[:, :1].astype(np.int64) - 127
    amax = np.abs(x).max(axis=1, keepdims=True)
    assert (np.exp2(e + 8) <= amax).all() and (amax < np.exp2(e + 9)).all()
    assert np.array_equal(c, torch_e4m3(np.ldexp(x, -e)))


def test_row_exponent_boundaries_saturation_and_zero():
    for amax, e in ((1.0, -8), (448.0, 0), (511.0, 0), (512.0, 1), (255.9, -1),
                    (2.0 ** 100, 92), (3.0 * 2.0 ** -120, -127)):
        row = np.zeros((1, 64))
        row[0, 40] = -amax
        row[0, 3] = amax / 5
        _, s = oracle.quant_fp8_rows(row)
        assert (s == e + 127).all(), (amax, s)
    c, s = oracle.quant_fp8_rows(np.array([[511.0, -470.0, -0.0] + [0.0] * 29]))
    assert (s == 127).all() and list(c[0, :3]) == [0x7E, 0xFE, 0x80]
    c, s = oracle.quant_fp8_rows(np.zeros((2, 32)))
    assert (s == 0).all() and not c.any()


def test_rows_whose_runs_share_the_exponent_equal_the_32_value_encoding():
    x = RNG.uniform(-1.0, 1.0, (30, 128))
    x[:, ::32] = np.where(RNG.random((30, 4)) < 0.5, -1.75, 1.75)  # each run max 1.75
    c, s = oracle.quant_fp8_rows(x)
    c32, s32 = oracle.quant_mxfp8(x)
    assert np.array_equal(s, s32) and np.array_equal(c, c32)


def test_scaling_by_a_power_of_two_shifts_only_the_exponent():
    x = RNG.standard_normal((20, 96))
    c, s = oracle.quant_fp8_rows(x)
    c2, s2 = oracle.quant_fp8_rows(x * 2.0 ** 13)
    assert np.array_equal(c, c2) and np.array_equal(s2.astype(int), s.astype(int) + 13)


def test_decoded_rows_are_within_half_a_step():
    x = RNG.standard_normal((40, 128)) * 2.5
    c, s = oracle.quant_fp8_rows(x)
    dq = oracle.dequant_mxfp8(c, s)
    e = s[:, :1].astype(np.int64) - 127
    y = np.abs(np.ldexp(x, -e))
    step = np.where(y < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(y, 1e-300))) - 3))
    sat = y > 448.0                          # saturated to 448
    assert (np.abs(dq - x)[~sat] <= np.ldexp(step / 2, e)[~sat]).all()
    assert (np.abs(dq[sat]) == np.ldexp(448.0, e.repeat(128, axis=1)[sat])).all()


def torch_weights(q, keys, scale):
    """Softmax weights [H, N] of one query [H, D] over keys [N, D] (torch, fp64)."""
    lg = torch.from_numpy(q) @ torch.from_numpy(keys).T * scale
    return torch.softmax(lg, dim=-1).numpy()


def test_stats_match_torch_softmax_weights():
    T, H, D, W, m, k = 90, 3, 16, 12, 4, 6
    K = RNG.standard_normal((1, T, D))
    V = RNG.standard_normal((1, T, D))
    ck = oracle.compress(K, RNG.standard_normal((1, T, D)), m)
    cv = oracle.compress(V, RNG.standard_normal((1, T, D)), m)
    q_pos = np.array([5, 40, 77, 89])
    q = RNG.standard_normal((1, len(q_pos), H, D))
    tk = np.full((1, len(q_pos), k), -1, np.int32)
    for i, t in enumerate(q_pos):
        n = oracle.n_cand(t, m, W)
        sel = RNG.permutation(n)[:min(k, n)]
        tk[0, i, :len(sel)] = np.sort(sel)
    o, am, rm = oracle.attend_stats(q, ck, cv, tk, K, V, 0, q_pos, m, W, scale=0.4)
    assert np.array_equal(o, oracle.attend(q, ck, cv, tk, K, V, 0, q_pos, m, W, scale=0.4))
    for i, t in enumerate(q_pos):
        w0 = max(0, t - W + 1)
        sel = [j for j in tk[0, i] if j >= 0]
        keys = np.concatenate([ck[0, sel], K[0, w0:t + 1]])
        vals = np.concatenate([cv[0, sel], V[0, w0:t + 1]])
        p = torch_weights(q[0, i], keys, 0.4)
        np.testing.assert_allclose(am[0, i], p @ np.abs(vals), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(rm[0, i], np.sqrt(p ** 2 @ vals ** 2), rtol=1e-12,
                                   atol=1e-14)
    # weighted means bound the output: |o| <= amean, rms <= amean
    assert (np.abs(o) <= am + 1e-12).all() and (rm <= am + 1e-12).all()


def test_stats_closed_forms():
    D, W = 8, 4
    V = RNG.standard_normal((1, 6, D))
    K = RNG.standard_normal((1, 6, D))
    z = np.zeros((1, 1, D))
    # one key (t = 0): the output is the value, both means are |v|
    o, am, rm = oracle.attend_stats(RNG.standard_normal((1, 1, 2, D)), z, z, None, K, V, 0,
                                    [0], 4, W)
    assert np.allclose(o[0, 0], V[0, 0]) and np.allclose(am[0, 0], np.abs(V[0, 0]))
    assert np.allclose(rm[0, 0], np.abs(V[0, 0]))
    # a zero query: equal weights 1/n over the window of n = 4 tokens (m = 8:
    # no complete block yet)
    o, am, rm = oracle.attend_stats(np.zeros((1, 1, 1, D)), z, z, None, K, V, 0, [5], 8, W)
    win = V[0, 2:6]
    np.testing.assert_allclose(am[0, 0, 0], np.abs(win).mean(axis=0), rtol=1e-13)
    np.testing.assert_allclose(rm[0, 0, 0], np.sqrt((win ** 2).sum(axis=0)) / 4, rtol=1e-13)


def test_attend_fp8_is_exact_attention_over_the_decoded_rows():
    B, T, H, D, W, m = 2, 70, 4, 128, 8, 4
    raw = RNG.standard_normal((B, T, D))
    ent = RNG.standard_normal((B, 17, D))
    q = RNG.standard_normal((B, 3, H, D)) * 0.1
    q_pos = np.array([9, 50, 69])
    enc = [oracle.quant_fp8_rows(a) for a in (ent, ent * 0.5, raw, raw * 2.0)]
    o, am, rm = oracle.attend_fp8(q, *enc[0], *enc[1], None, *enc[2], *enc[3], 0, q_pos, m, W)
    dec = [oracle.dequant_mxfp8(c, s) for c, s in enc]
    qhat = oracle.dequant_mxfp8(*oracle.quant_fp8_rows(q))
    ref = oracle.attend_stats(qhat, dec[0], dec[1], None, dec[2], dec[3], 0, q_pos, m, W)
    for a, b in zip((o, am, rm), ref):
        assert np.array_equal(a, b)
    # queries already on their rows' FP8 grid are used unchanged
    o2, _, _ = oracle.attend_fp8(qhat, *enc[0], *enc[1], None, *enc[2], *enc[3], 0, q_pos, m, W)
    assert np.array_equal(o2, o)
    # and the whole reading stays within a few FP8 steps of attention on the
    # unencoded values
    exact = oracle.attend(q, ent, ent * 0.5, None, raw, raw * 2.0, 0, q_pos, m, W)
    assert np.abs(o - exact).max() < 0.1 * np.abs(exact).max()


@pytest.mark.parametrize("d", [31, 0])
def test_rejects_bad_width(d):
    with pytest.raises(ValueError):
        oracle.quant_fp8_rows(np.zeros((2, d)))
