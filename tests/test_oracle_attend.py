"""Pins of the oracle's attention step (jiwasawa.github.io post: CSA "Shared
Key-Value MQA" over the selected entries, HCA dense attention over every
compressed entry, SWA branch over the newest tokens; hazakura.dev note, CSA
and HCA bullets).

Every case is compared with torch's scaled_dot_product_attention on the CPU
in float64 with an explicit mask: causal attention (m=1, all candidates
kept), sliding-window attention (nothing kept), dense compressed attention
(k >= candidates) and the general sparse case over a concatenated key set.
Also a two-key logistic closed form and invariance to the order of the
selected slots."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(5)


def sdpa(q, keys, vals, allow, scale):
    """q [Tq,H,D], keys/vals [N,D], allow [Tq,N] bool -> [Tq,H,D]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]              # [1,H,Tq,D]
    kt = torch.from_numpy(keys)[None, None].expand(1, q.shape[1], -1, -1)
    vt = torch.from_numpy(vals)[None, None].expand(1, q.shape[1], -1, -1)
    mask = torch.from_numpy(allow)[None, None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def all_candidates(q_pos, m, W, k):
    tk = np.full((1, len(q_pos), k), -1, np.int32)
    for i, t in enumerate(q_pos):
        n = oracle.n_cand(t, m, W)
        assert n <= k
        tk[0, i, :n] = np.arange(n)
    return tk


@pytest.mark.parametrize("W", [0, 1, 5, 16])
def test_m1_all_kept_is_causal_attention(W):
    T, H, D = 40, 3, 8
    K = RNG.standard_normal((1, T, D))
    V = RNG.standard_normal((1, T, D))
    q_pos = np.arange(T)
    q = RNG.standard_normal((1, T, H, D))
    ck, cv = oracle.compress(K, np.zeros((1, T, 1)), 1), oracle.compress(V, np.zeros((1, T, 1)), 1)
    tk = all_candidates(q_pos, 1, W, T)
    o = oracle.attend(q, ck, cv, tk, K, V, 0, q_pos, 1, W, scale=0.3)
    ref = sdpa(q[0], K[0], V[0], np.tril(np.ones((T, T), bool)), 0.3)
    np.testing.assert_allclose(o[0], ref, rtol=1e-12, atol=1e-12)
    # HCA with m' = 1 is the same causal attention
    o2 = oracle.attend(q, ck, cv, None, K, V, 0, q_pos, 1, W, scale=0.3)
    np.testing.assert_allclose(o2[0], ref, rtol=1e-12, atol=1e-12)


def test_nothing_kept_is_sliding_window_attention():
    T, H, D, W, m = 64, 2, 8, 9, 4
    K = RNG.standard_normal((1, T, D))
    V = RNG.standard_normal((1, T, D))
    q = RNG.standard_normal((1, T, H, D))
    q_pos = np.arange(T)
    ck = RNG.standard_normal((1, T // m, D))
    cv = RNG.standard_normal((1, T // m, D))
    tk = np.full((1, T, 4), -1, np.int32)
    o = oracle.attend(q, ck, cv, tk, K, V, 0, q_pos, m, W)
    i = np.arange(T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)
    np.testing.assert_allclose(o[0], sdpa(q[0], K[0], V[0], band, 1.0), rtol=1e-12, atol=1e-12)


def general_reference(q, ck, cv, tk, rk, rv, raw_pos0, q_pos, m, W, scale):
    """Keys = [compressed entries ; raw rows]; row i may see the compressed
    entries named in its first min(k, n_cand) slots and the raw rows of its
    window."""
    Nc, R = ck.shape[1], rk.shape[1]
    allow = np.zeros((len(q_pos), Nc + R), bool)
    for i, t in enumerate(q_pos):
        nc = oracle.n_cand(t, m, W)
        if tk is None:
            allow[i, :nc] = True
        else:
            for j in tk[0, i, :min(tk.shape[2], nc)]:
                if 0 <= j < nc:
                    allow[i, j] = True
        w0 = max(0, t - W + 1)
        allow[i, Nc + (w0 - raw_pos0):Nc + (t - raw_pos0) + 1] = True
    keys = np.concatenate([ck[0], rk[0]])
    vals = np.concatenate([cv[0], rv[0]])
    return sdpa(q[0], keys, vals, allow, scale)


@pytest.mark.parametrize("m,W,k", [(4, 16, 6), (4, 128, 512), (3, 7, 2), (128, 128, 0)])
def test_general_sparse_case_against_masked_sdpa(m, W, k):
    T, H, D = 700, 4, 16
    Nc = T // m
    q_pos = np.array(sorted(RNG.choice(np.arange(T), size=12, replace=False)))
    q = RNG.standard_normal((1, len(q_pos), H, D))
    ck = RNG.standard_normal((1, Nc, D))
    cv = RNG.standard_normal((1, Nc, D))
    rk = RNG.standard_normal((1, T, D))
    rv = RNG.standard_normal((1, T, D))
    if k == 0:
        tk = None                     # HCA: every candidate
    else:
        tk = np.full((1, len(q_pos), k), -1, np.int32)
        for i, t in enumerate(q_pos):
            n = oracle.n_cand(t, m, W)
            sel = np.sort(RNG.choice(n, size=min(k, n), replace=False)) if n else []
            tk[0, i, :len(sel)] = sel
    o = oracle.attend(q, ck, cv, tk, rk, rv, 0, q_pos, m, W, scale=0.7)
    ref = general_reference(q, ck, cv, tk, rk, rv, 0, q_pos, m, W, 0.7)
    np.testing.assert_allclose(o[0], ref, rtol=1e-11, atol=1e-12)


def test_decode_window_only_raw_tail():
    # raw rows only cover the last W positions; positions are offset
    m, W, H, D, Nc = 4, 8, 2, 8, 300
    t = 4 * Nc - 1
    q = RNG.standard_normal((1, 1, H, D))
    ck = RNG.standard_normal((1, Nc, D))
    cv = RNG.standard_normal((1, Nc, D))
    rk = RNG.standard_normal((1, W, D))
    rv = RNG.standard_normal((1, W, D))
    raw_pos0 = t - W + 1
    o = oracle.attend(q, ck, cv, None, rk, rv, raw_pos0, [t], m, W)
    ref = general_reference(q, ck, cv, None, rk, rv, raw_pos0, [t], m, W, 1.0)
    np.testing.assert_allclose(o[0], ref, rtol=1e-11, atol=1e-12)
    with pytest.raises(ValueError):          # window not covered by raw rows
        oracle.attend(q, ck, cv, None, rk[:, 1:], rv[:, 1:], raw_pos0 + 1, [t], m, W)


def test_two_keys_logistic_closed_form():
    # t = 0 with W >= 1: only the raw key 0 -> output equals v0
    # t = 1, W = 2, no compressed: softmax of two logits
    D = 4
    rk = RNG.standard_normal((1, 2, D))
    rv = RNG.standard_normal((1, 2, D))
    q = RNG.standard_normal((1, 1, 1, D))
    ck = np.zeros((1, 0, D))
    o = oracle.attend(q, ck, ck, None, rk, rv, 0, [1], 4, 2)
    l0, l1 = q[0, 0, 0] @ rk[0, 0], q[0, 0, 0] @ rk[0, 1]
    ref = rv[0, 0] / (1 + np.exp(l1 - l0)) + rv[0, 1] / (1 + np.exp(l0 - l1))
    np.testing.assert_allclose(o[0, 0, 0], ref, rtol=1e-13, atol=1e-14)


def test_slot_order_does_not_matter():
    m, W, H, D, T = 4, 16, 2, 8, 400
    Nc = T // m
    q = RNG.standard_normal((1, 1, H, D))
    ck = RNG.standard_normal((1, Nc, D))
    cv = RNG.standard_normal((1, Nc, D))
    rk = RNG.standard_normal((1, T, D))
    rv = RNG.standard_normal((1, T, D))
    t = T - 1
    sel = np.sort(RNG.choice(oracle.n_cand(t, m, W), size=10, replace=False)).astype(np.int32)
    a = oracle.attend(q, ck, cv, sel[None, None], rk, rv, 0, [t], m, W)
    b = oracle.attend(q, ck, cv, sel[::-1].copy()[None, None], rk, rv, 0, [t], m, W)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_slots_past_candidate_count_are_ignored():
    m, W, H, D, T = 4, 16, 2, 8, 200
    Nc = T // m
    q = RNG.standard_normal((1, 1, H, D))
    ck = RNG.standard_normal((1, Nc, D))
    cv = RNG.standard_normal((1, Nc, D))
    rk = RNG.standard_normal((1, T, D))
    rv = RNG.standard_normal((1, T, D))
    t = 40                                      # n_cand = 7
    assert oracle.n_cand(t, m, W) == 7
    tk = np.array([[[0, 3, 6, 1, 2, 4, 5, 9, 11]]], np.int32)   # slots 7, 8 ignored
    a = oracle.attend(q, ck, cv, tk, rk, rv, 0, [t], m, W)
    b = oracle.attend(q, ck, cv, None, rk, rv, 0, [t], m, W)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
