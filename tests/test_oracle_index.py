"""Pins of the oracle's candidate set, Lightning Indexer score and top-k
selector (jiwasawa.github.io post, CSA indexer bullet; studioglobal.ai
answer, CSA bullet: FP4 indexer keeps the top 512 compressed blocks per
query; hazakura.dev note, CSA bullets: 128-token sliding window).

The score is checked against a float64 matmul of independently dequantised
values; the selection against a brute-force characterisation of the top-k
set (every kept entry beats every dropped one); the candidate count against
a hand-derived table (tests/golden/n_cand.json)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from tests.test_oracle_mxfp4 import decode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "n_cand.json")
RNG = np.random.default_rng(99)


def test_candidate_count_table():
    for t, m, W, n in json.load(open(GOLDEN))["cases"]:
        assert oracle.n_cand(t, m, W) == n, (t, m, W)


def test_candidate_count_closed_form():
    # for W >= m-1 a block that starts before the window is complete, so the
    # count is ceil(w0 / m)
    for m in (1, 2, 4, 16, 128):
        for W in (m - 1, 128, 300):
            for t in list(range(0, 400, 7)) + [4095, 65536 + 13]:
                w0 = max(0, t - W + 1)
                assert oracle.n_cand(t, m, W) == -(-w0 // m)


def ref_scores(q_idx, k_idx, q_pos, m, W):
    """sum_h relu(dequant(q_h) . dequant(k)) by a float64 matmul."""
    qc, qs = oracle.quant_mxfp4(q_idx)
    kc, ks = oracle.quant_mxfp4(k_idx)
    B, Tq, HI, dI = q_idx.shape
    qd = decode(qc, qs, dI)
    kd = decode(kc, ks, dI)
    s = np.einsum("bthd,bnd->bthn", qd, kd)
    s = np.maximum(s, 0).sum(axis=2)
    for i, t in enumerate(q_pos):
        s[:, i, oracle.n_cand(t, m, W):] = -1
    return s, (qc, qs, kc, ks)


@pytest.mark.parametrize("HI,dI", [(1, 32), (2, 32), (4, 64)])
def test_scores_equal_dequantised_matmul(HI, dI):
    B, Tq, Nc, m, W = 2, 5, 45, 4, 16
    q_idx = RNG.standard_normal((B, Tq, HI, dI))
    k_idx = RNG.standard_normal((B, Nc, dI))
    q_pos = np.array([3, 70, 100, 150, 179])
    ref, (qc, qs, kc, ks) = ref_scores(q_idx, k_idx, q_pos, m, W)
    got, exact = oracle.index_scores(qc, qs, kc, ks, q_pos, m, W)
    assert exact
    assert np.array_equal(got.astype(np.float64), ref)


def test_relu_per_head_before_sum():
    # head 0 anti-aligned with the key, head 1 aligned: score = head 1 only
    dI = 32
    k = np.zeros((1, 1, dI)); k[0, 0, 0] = 1.0
    q = np.zeros((1, 1, 2, dI)); q[0, 0, 0, 0] = -3.0; q[0, 0, 1, 0] = 2.0
    qc, qs = oracle.quant_mxfp4(q)
    kc, ks = oracle.quant_mxfp4(k)
    s, exact = oracle.index_scores(qc, qs, kc, ks, [128], 4, 128)
    assert exact and s[0, 0, 0] == 2.0
    q[0, 0, 1, 0] = -1.0      # both heads negative -> +0
    qc, qs = oracle.quant_mxfp4(q)
    s, _ = oracle.index_scores(qc, qs, kc, ks, [128], 4, 128)
    assert s[0, 0, 0] == 0.0 and not np.signbit(s[0, 0, 0])


def test_exactness_guard_trips_on_wide_scale_span():
    dI = 64
    q = np.zeros((1, 1, 1, dI)); q[0, 0, 0, :32] = 6.0 * 2.0 ** 20; q[0, 0, 0, 32] = 0.5
    k = np.zeros((1, 1, dI)); k[0, 0, :32] = 6.0 * 2.0 ** 20; k[0, 0, 32] = 0.5
    qc, qs = oracle.quant_mxfp4(q)
    kc, ks = oracle.quant_mxfp4(k)
    _, exact = oracle.index_scores(qc, qs, kc, ks, [128], 4, 128)
    assert not exact


def test_gaussian_inputs_are_exact_in_fp32():
    q = RNG.standard_normal((1, 4, 4, 64))
    k = RNG.standard_normal((1, 300, 64))
    qc, qs = oracle.quant_mxfp4(q)
    kc, ks = oracle.quant_mxfp4(k)
    _, exact = oracle.index_scores(qc, qs, kc, ks, [1300, 1301, 1302, 1303], 4, 128)
    assert exact


def brute_topk(row, nc, k):
    """The unique set S of size min(k, nc) of candidates such that every member
    beats every non-member under (score desc, index asc), by enumeration."""
    n = min(k, nc)
    beats = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)
    found = [S for S in itertools.combinations(range(nc), n)
             if all(beats(a, b) for a in S for b in range(nc) if b not in S)]
    assert len(found) == 1
    return list(found[0]) + [-1] * (k - n)


def test_topk_brute_force_with_ties():
    for trial in range(30):
        nc = int(RNG.integers(0, 9))
        k = int(RNG.integers(1, 6))
        Nc = 10
        row = RNG.choice([0.0, 0.5, 1.0, 2.0], size=Nc).astype(np.float32)
        scores = row[None, None, :]
        t = 4 * nc + 127 if nc else 0          # m=4, W=128 -> exactly nc candidates
        assert oracle.n_cand(t, 4, 128) == nc
        got = oracle.select_topk(scores, [t], 4, 128, k)
        assert got[0, 0].tolist() == brute_topk(row, nc, k)


def test_tie_storm_keeps_lowest_indices():
    Nc, k = 600, 512
    scores = np.full((1, 1, Nc), 3.0, np.float32)
    t = oracle_t = 4 * Nc + 127
    got = oracle.select_topk(scores, [t], 4, 128, k)
    assert got[0, 0].tolist() == list(range(k))


def test_fewer_candidates_than_k_pads():
    scores = RNG.standard_normal((1, 1, 50)).astype(np.float32)
    t = 4 * 20 + 127
    got = oracle.select_topk(np.abs(scores), [t], 4, 128, 32)
    assert got[0, 0, :20].tolist() == list(range(20))
    assert (got[0, 0, 20:] == -1).all()


def test_non_candidates_never_selected():
    scores = np.zeros((1, 1, 64), np.float32)
    scores[0, 0, 40:] = 100.0                  # beyond n_cand
    t = 4 * 30 + 127
    got = oracle.select_topk(scores, [t], 4, 128, 8)
    assert got[0, 0].tolist() == list(range(8))


def test_union_of_chunk_topk_is_global_topk():
    Nc, k, C = 4096, 64, 512
    row = RNG.choice(np.arange(40, dtype=np.float32) / 4, size=Nc)
    t = 4 * Nc + 127
    full = oracle.select_topk(row[None, None], [t], 4, 128, k)[0, 0]
    keep = []
    for c0 in range(0, Nc, C):
        sub = oracle.select_topk(row[None, None, c0:c0 + C], [4 * C + 127], 4, 128, k)[0, 0]
        keep += [c0 + j for j in sub if j >= 0]
    keep = np.array(keep)
    merged = oracle.select_topk(row[keep][None, None], [4 * len(keep) + 127], 4, 128, k)[0, 0]
    assert np.array_equal(np.sort(keep[merged]), full)


def test_index_topk_matches_scores_then_select():
    B, Tq, HI, dI, Nc, m, W, k = 2, 6, 4, 64, 300, 4, 128, 16
    q = RNG.standard_normal((B, Tq, HI, dI))
    kk = RNG.standard_normal((B, Nc, dI))
    kc, ks = oracle.quant_mxfp4(kk)
    qc, qs = oracle.quant_mxfp4(q)
    q_pos = np.array([0, 130, 500, 900, 1199, 1327])
    s, ex1 = oracle.index_scores(qc, qs, kc, ks, q_pos, m, W)
    a = oracle.select_topk(s, q_pos, m, W, k)
    b, ex2 = oracle.index_topk(q, kc, ks, q_pos, m, W, k)
    assert ex1 and ex2
    assert np.array_equal(a, b)
