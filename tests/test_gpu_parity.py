"""GPU parity of every step against the CPU oracle, on the same seeded
inputs, through the C ABI (ctypes binding).

Bars: MXFP4 codes/scales and top-k indices bit-exact; values within max-abs
1e-5 (fp32) and 2e-2 (bf16).  Sizes span several tiles/chunks with ragged
tails; edge cases: candidate counts below k, tie storms, one-chunk and
multi-chunk selection, decode with split key lists, m = 1, m = 128."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from compressed_sparse_attention_04_amd import binding as csa
from compressed_sparse_attention_04_amd import inputs as I
from tests.gpu_helpers import DEV, TOL, f64, maxerr, random_selection, say

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- compress
@pytest.mark.parametrize("dtype,C,m,T,B,gate", [
    ("f32", 64, 4, 1024, 1, "token"),
    ("bf16", 128, 4, 1001, 2, "channel"),
    ("bf16", 128, 128, 128 * 9 + 57, 2, "channel"),
    ("f32", 64, 128, 128 * 5, 1, "channel"),
    ("bf16", 128, 16, 16 * 33, 1, "token"),
    ("bf16", 64, 17, 17 * 21 + 3, 3, "channel"),
    ("bf16", 128, 1, 300, 1, "channel"),
])
def test_compress(dtype, C, m, T, B, gate):
    say("compress", dtype, C, m, T, B, gate)
    w = I.Workload("t", "csa", seed=11, dtype=dtype, B=B, T=T, m=m, H=8, D=C, gate=gate)
    raw = I.draw_raw(w)
    ref_k = oracle.compress(f64(raw["k"]), f64(raw["gk"]), m)
    got = csa.hca_compress(raw["k"].to(DEV), raw["gk"].to(DEV), m)
    torch.cuda.synchronize()
    err = maxerr(got, ref_k)
    say("  max err", err)
    assert err <= TOL[dtype]
    if m == 1:
        assert torch.equal(got.cpu(), raw["k"])


# ---------------------------------------------------------------- MXFP4
def quant_inputs(rng, rows, d):
    x = rng.standard_normal((rows, d)) * np.exp(rng.uniform(-8, 8, size=(rows, 1)))
    x[0] = 0.0
    x[1, :] = 0.0
    x[1, 3] = -0.0
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                        "mxfp4_rounding.json")))["cases"]
    for r, (v, _) in enumerate(cases[: rows - 4]):
        x[r + 2, :] = 0.0
        x[r + 2, 0] = v
        x[r + 2, 5] = 6.0
        x[r + 2, 9] = -v / 2
    x[-1, :32] = np.ldexp(rng.standard_normal(32), -140)   # fp32 subnormals
    return x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_bit_exact(dtype):
    say("quantize", dtype)
    rng = np.random.default_rng(3)
    x = torch.from_numpy(quant_inputs(rng, 256, 64)).to(I.torch_dtype(dtype))
    if dtype == "bf16":
        x[-1] = 0          # bf16 has no fp32-subnormal range worth testing here
    ref_c, ref_s = oracle.quant_mxfp4(f64(x))
    c, s = csa.csa_quantize_mxfp4(x.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), ref_s)
    assert np.array_equal(c.cpu().numpy(), ref_c)


# ---------------------------------------------------------------- indexer
def index_case(w: I.Workload, q_pos0: int, Tq: int, tie=False):
    w = w.replace(Tq=Tq, q_pos0=q_pos0)
    k_idx = I.draw_indexer_keys(w)
    if tie:
        k_idx[:] = k_idx[:, :1]
    q_idx = I.draw_indexer_queries(w)
    kc, ks = oracle.quant_mxfp4(f64(k_idx))
    q_pos = np.arange(q_pos0, q_pos0 + Tq)
    ref, exact = oracle.index_topk(f64(q_idx), kc, ks, q_pos, w.m, w.W, w.k)
    assert exact
    gkc, gks = csa.csa_quantize_mxfp4(k_idx.to(DEV))
    got = csa.csa_index_topk(q_idx.to(DEV), gkc, gks, m=w.m, W=w.W, k=w.k, q_pos0=q_pos0)
    torch.cuda.synchronize()
    assert np.array_equal(gkc.cpu().numpy(), kc) and np.array_equal(gks.cpu().numpy(), ks)
    g = got.cpu().numpy()
    bad = np.argwhere((g != ref).any(axis=2))
    assert bad.size == 0, f"{len(bad)} rows differ, first {bad[:3].tolist()}"
    return g


def test_index_tiny_config():
    say("index tiny")
    w = I.TINY_CSA
    index_case(w, w.q_pos0, w.Tq)


@pytest.mark.parametrize("T,q_pos0,Tq,B", [
    (4096, 0, 37, 1),              # early rows: no candidates / fewer than k
    (12000, 2200, 45, 2),          # around the k-saturation point, one chunk
    (12000, 11950, 50, 1),         # 2955+ candidates, one chunk
])
def test_index_bf16_one_chunk(T, q_pos0, Tq, B):
    say("index one chunk", T, q_pos0, Tq, B)
    w = I.Workload("t", "csa", seed=21, dtype="bf16", B=B, T=T, m=4, H=128, D=128)
    index_case(w, q_pos0, Tq)


@pytest.mark.parametrize("T,q_pos0,Tq,B,k", [
    # streaming path (candidates <= 32768 per block of 8 rows)
    (40000, 39990, 10, 2, 512),
    (40000, 16500, 9, 1, 300),
    (4 * 32768, 4 * 32768 - 20, 20, 1, 512),   # largest streaming candidate count
    (40000, 39990, 10, 1, 768),    # largest k of the sampled path
    (40000, 39990, 10, 1, 1000),   # k above it: exact search, read-out staged in LDS
    (40000, 39990, 10, 1, 1500),   # k above the staging room: direct read-out
    # decode path (<= 8 rows, > 4096 candidates): chunked scores + select
    (4 * 70000, 4 * 70000 - 1, 1, 3, 512),
    (4 * 50000, 4 * 50000 - 8, 8, 2, 512),
    (4 * 262144, 4 * 262144 - 1, 1, 2, 512),   # 1M-token context row
    (4 * 5000, 4 * 5000 - 3, 3, 1, 2048),
    # chunk + merge path (> 8 rows with > 32768 candidates)
    (140000, 139990, 10, 1, 512),
])
def test_index_bf16_paths(T, q_pos0, Tq, B, k):
    say("index paths", T, q_pos0, Tq, B, k)
    w = I.Workload("t", "csa", seed=22, dtype="bf16", B=B, T=T, m=4, H=128, D=128, k=k)
    index_case(w, q_pos0, Tq)


@pytest.mark.parametrize("T,q_pos0,Tq", [(3000, 2900, 8), (40000, 39990, 3), (40000, 39990, 9),
                                         (140000, 139990, 10)])
def test_index_tie_storm_keeps_lowest(T, q_pos0, Tq):
    say("index tie storm", T, q_pos0, Tq)
    w = I.Workload("t", "csa", seed=23, dtype="bf16", B=1, T=T, m=4, H=128, D=128)
    g = index_case(w, q_pos0, Tq, tie=True)
    for i in range(Tq):
        # all keys equal: scores equal within a query -> indices 0..k-1
        assert g[0, i].tolist() == list(range(512))


@pytest.mark.parametrize("T,q_pos0,Tq,shrink", [(40000, 39990, 10, True), (40000, 39990, 10, False),
                                                (20000, 19000, 16, True)])
def test_index_unrepresentative_sample(T, q_pos0, Tq, shrink):
    """Keys of every 8th tile of 32 (j % 256 < 32) scaled by 1/64 (or 64):
    a range estimated from those tiles alone misses the k-th key, so the
    exact search must take over and still give the oracle's set."""
    say("index skewed sample", T, q_pos0, Tq, shrink)
    w = I.Workload("t", "csa", seed=25, dtype="bf16", B=1, T=T, m=4, H=128, D=128)
    w = w.replace(Tq=Tq, q_pos0=q_pos0)
    k_idx = I.draw_indexer_keys(w)
    j = torch.arange(k_idx.shape[1])
    f = 1.0 / 64 if shrink else 64.0
    k_idx[:, (j % 256) < 32] = (k_idx[:, (j % 256) < 32].float() * f).to(k_idx.dtype)
    q_idx = I.draw_indexer_queries(w)
    kc, ks = oracle.quant_mxfp4(f64(k_idx))
    q_pos = np.arange(q_pos0, q_pos0 + Tq)
    ref, exact = oracle.index_topk(f64(q_idx), kc, ks, q_pos, w.m, w.W, w.k)
    assert exact
    gkc, gks = csa.csa_quantize_mxfp4(k_idx.to(DEV))
    got = csa.csa_index_topk(q_idx.to(DEV), gkc, gks, m=w.m, W=w.W, k=w.k, q_pos0=q_pos0)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("copies", [600, 100, 40])
def test_index_decode_clustered_range(copies):
    """Decode path: the keys around the k-th score all sit in one chunk of
    4096 candidates (copies of the row's best key, with 300 keys at twice
    its score elsewhere), more than that chunk's buffer slots hold when
    copies = 600: the final kernel must rescan and still keep the lowest
    indices of the tie."""
    say("index clustered range", copies)
    w = I.Workload("t", "csa", seed=26, dtype="bf16", B=1, T=4 * 70000, m=4, H=128, D=128)
    q_pos0 = 4 * 70000 - 1
    w = w.replace(Tq=1, q_pos0=q_pos0)
    k_idx = I.draw_indexer_keys(w)
    q_idx = I.draw_indexer_queries(w)
    q_pos = np.array([q_pos0])
    kc, ks = oracle.quant_mxfp4(f64(k_idx))
    qc, qs = oracle.quant_mxfp4(f64(q_idx))
    sc, _ = oracle.index_scores(qc, qs, kc, ks, q_pos, w.m, w.W)
    best = int(np.argmax(sc[0, 0, :oracle.n_cand(q_pos0, w.m, w.W)]))
    k_idx[:, 8192:8192 + copies] = k_idx[:, best:best + 1]
    k_idx[:, 20000:20300] = k_idx[:, best:best + 1] * 2          # exactly twice the score
    kc, ks = oracle.quant_mxfp4(f64(k_idx))
    ref, exact = oracle.index_topk(f64(q_idx), kc, ks, q_pos, w.m, w.W, w.k)
    assert exact
    gkc, gks = csa.csa_quantize_mxfp4(k_idx.to(DEV))
    got = csa.csa_index_topk(q_idx.to(DEV), gkc, gks, m=w.m, W=w.W, k=w.k, q_pos0=q_pos0)
    torch.cuda.synchronize()
    g = got.cpu().numpy()
    assert np.array_equal(g, ref)
    assert set(range(20000, 20300)) <= set(g[0, 0].tolist())


@pytest.mark.parametrize("dtype,HI,dI,T,Tq,B,k", [
    ("f32", 2, 64, 4 * 60000, 2, 2, 512),
    ("bf16", 1, 32, 4 * 100000, 5, 1, 256),
    ("bf16", 4, 32, 4 * 262144, 8, 1, 512),      # 256 chunks of 1024, 32 list slots each
    ("bf16", 4, 64, 4 * 262144, 1, 1, 2048),     # 64 chunks, 128 list slots, k = 2048
    ("bf16", 2, 64, 4 * 9000, 4, 3, 64),
])
def test_index_decode_shapes(dtype, HI, dI, T, Tq, B, k):
    """Decode path (<= 8 rows, > 4096 candidates) at every indexer head count,
    both indexer dims, fp32 and bf16 queries, 1 to 8 rows, and chunk
    geometries from 4096 to 1024 candidates: chunk lists merged exactly."""
    say("index decode shapes", dtype, HI, dI, T, Tq, B, k)
    w = I.Workload("t", "csa", seed=27, dtype=dtype, B=B, T=T, m=4, H=128, D=128, HI=HI, dI=dI,
                   k=k)
    index_case(w, T - Tq, Tq)


def test_index_one_head_small_k():
    say("index HI=1")
    w = I.Workload("t", "csa", seed=24, dtype="f32", B=2, T=6000, m=4, H=8, D=64, HI=1, dI=64,
                   k=64)
    index_case(w, 5000, 70)


# ---------------------------------------------------------------- attention
def attend_case(dtype, H, D, T, m, W, k, q_rows, B=1, seed=31, decode_tail=False, corrupt=False,
                shared_kv=False):
    """Stage-wise: q, compressed and raw caches drawn directly; kept sets
    drawn at random (k > 0) or every candidate (k == 0, HCA).  corrupt: about
    one kept entry in eight replaced by -1 or an index past the candidates
    (entries that contribute nothing).  shared_kv: one vector per entry and
    raw token serves as key and value (the same device buffers passed as K
    and V)."""
    w = I.Workload("t", "csa", seed=seed, dtype=dtype, B=B, T=T, m=m, H=H, D=D, W=W, k=max(k, 1),
                   Tq=len(q_rows), q_pos0=int(q_rows[0]))
    Nc = T // m
    q = I.draw_queries(w)
    ck = I.draw_cache(w, "ck", Nc)
    cv = I.draw_cache(w, "cv", Nc)
    if decode_tail:
        raw_pos0 = int(q_rows[0]) - W + 1
        rk = I.draw_cache(w, "rk", W)
        rv = I.draw_cache(w, "rv", W)
    else:
        raw_pos0 = 0
        rk = I.draw_cache(w, "rk", T)
        rv = I.draw_cache(w, "rv", T)
    if shared_kv:
        cv, rv = ck, rk
    q_pos = np.asarray(q_rows)
    d_ck, d_rk = ck.to(DEV), rk.to(DEV)
    d_cv = d_ck if shared_kv else cv.to(DEV)
    d_rv = d_rk if shared_kv else rv.to(DEV)
    rng = np.random.default_rng(seed)
    if k > 0:
        tk = np.array([[random_selection(rng, oracle.n_cand(t, m, W), k) for t in q_pos]
                       for _ in range(B)], np.int32)
        if corrupt:
            nc = np.array([oracle.n_cand(t, m, W) for t in q_pos])
            bad = rng.random(tk.shape) < 0.125
            junk = np.where(rng.random(tk.shape) < 0.5, -1, nc[None, :, None] + 3)
            tk = np.where(bad, junk, tk).astype(np.int32)
        ref = oracle.attend(f64(q), f64(ck), f64(cv), tk, f64(rk), f64(rv), raw_pos0, q_pos, m, W)
        got = csa.csa_attend(q.to(DEV), d_ck, d_cv, torch.from_numpy(tk).to(DEV), d_rk, d_rv,
                             m=m, W=W, q_pos0=int(q_pos[0]), raw_pos0=raw_pos0)
    else:
        ref = oracle.attend(f64(q), f64(ck), f64(cv), None, f64(rk), f64(rv), raw_pos0, q_pos, m,
                            W)
        got = csa.hca_attend(q.to(DEV), d_ck, d_cv, d_rk, d_rv, m=m, W=W, q_pos0=int(q_pos[0]),
                             raw_pos0=raw_pos0)
    torch.cuda.synchronize()
    err = maxerr(got, ref)
    say("  max err", err)
    assert err <= TOL[dtype]


def rows(a, n):
    return list(range(a, a + n))


@pytest.mark.parametrize("case", [
    dict(dtype="f32", H=8, D=64, T=1024, m=4, W=128, k=16, q_rows=rows(1008, 16)),
    dict(dtype="f32", H=3, D=40, T=300, m=4, W=16, k=5, q_rows=rows(0, 70)),
    dict(dtype="bf16", H=128, D=128, T=3000, m=4, W=128, k=64, q_rows=rows(0, 5) + []),
    dict(dtype="bf16", H=128, D=128, T=3000, m=4, W=128, k=64, q_rows=rows(2900, 33)),
    dict(dtype="bf16", H=128, D=128, T=6000, m=4, W=128, k=512, q_rows=rows(5500, 9), B=2),
    dict(dtype="bf16", H=32, D=64, T=2000, m=4, W=40, k=100, q_rows=rows(1000, 17)),
    dict(dtype="bf16", H=128, D=64, T=2500, m=4, W=100, k=200, q_rows=rows(1, 51)),
    dict(dtype="bf16", H=256, D=128, T=2000, m=4, W=128, k=32, q_rows=rows(1900, 3)),
])
def test_csa_attend(case):
    say("csa_attend", case)
    attend_case(**case)


@pytest.mark.parametrize("case", [
    dict(dtype="f32", H=4, D=64, T=2000, m=128, W=128, k=0, q_rows=rows(1900, 20)),
    dict(dtype="bf16", H=128, D=128, T=5000, m=128, W=128, k=0, q_rows=rows(4950, 40)),
    dict(dtype="bf16", H=128, D=128, T=700, m=4, W=64, k=0, q_rows=rows(0, 30)),
    dict(dtype="bf16", H=128, D=64, T=3000, m=16, W=128, k=0, q_rows=rows(2000, 37)),
])
def test_hca_attend(case):
    say("hca_attend", case)
    attend_case(**case)


# Many query rows (>= 512): one block per row, no split of the key list;
# rows from position 0 have one-tile key lists, and a corrupted kept list
# has invalid entries in the middle of its tiles.
@pytest.mark.parametrize("case", [
    dict(dtype="bf16", H=128, D=128, T=3000, m=4, W=128, k=64, q_rows=rows(0, 600)),
    dict(dtype="bf16", H=128, D=128, T=5000, m=4, W=128, k=512, q_rows=rows(4400, 600)),
    dict(dtype="bf16", H=128, D=64, T=2500, m=4, W=100, k=200, q_rows=rows(1500, 300), B=2),
    dict(dtype="bf16", H=256, D=128, T=2000, m=4, W=128, k=32, q_rows=rows(1400, 520)),
    dict(dtype="bf16", H=256, D=64, T=2000, m=4, W=128, k=48, q_rows=rows(1000, 530)),
    dict(dtype="bf16", H=128, D=128, T=3000, m=4, W=128, k=100, q_rows=rows(2000, 700),
         corrupt=True),
    dict(dtype="bf16", H=128, D=128, T=1200, m=4, W=64, k=0, q_rows=rows(0, 1100)),
    dict(dtype="bf16", H=128, D=64, T=3000, m=16, W=128, k=0, q_rows=rows(2200, 400), B=2),
    dict(dtype="bf16", H=256, D=128, T=5000, m=128, W=128, k=0, q_rows=rows(4400, 600)),
])
def test_attend_many_rows(case):
    say("attend many rows", case)
    attend_case(**case)


# One vector as key and value (the shared key-value reading): the library
# copies each row once and reads the value operands from the key tiles.
@pytest.mark.parametrize("case", [
    dict(dtype="bf16", H=128, D=128, T=3000, m=4, W=128, k=64, q_rows=rows(2900, 33)),
    dict(dtype="bf16", H=128, D=128, T=3000, m=4, W=128, k=100, q_rows=rows(2000, 600),
         corrupt=True),
    dict(dtype="bf16", H=64, D=64, T=2000, m=4, W=40, k=100, q_rows=rows(1000, 17)),
    dict(dtype="bf16", H=128, D=128, T=1200, m=4, W=64, k=0, q_rows=rows(0, 700)),
    dict(dtype="bf16", H=256, D=64, T=3000, m=16, W=128, k=0, q_rows=rows(2000, 37)),
    dict(dtype="bf16", H=128, D=128, T=128 * 3000, m=128, W=128, k=0, q_rows=[128 * 3000 - 1],
         B=3, decode_tail=True),
    dict(dtype="bf16", H=128, D=128, T=4 * 20000, m=4, W=128, k=512, q_rows=[4 * 20000 - 1],
         B=2, decode_tail=True),
    dict(dtype="f32", H=8, D=64, T=1024, m=4, W=128, k=16, q_rows=rows(1008, 16)),
])
def test_attend_shared_kv(case):
    say("attend shared kv", case)
    attend_case(shared_kv=True, **case)


@pytest.mark.parametrize("case", [
    # decode rows: one query per sequence, raw rows hold only the window,
    # the key list is split over blocks and merged
    dict(dtype="bf16", H=128, D=128, T=128 * 3000, m=128, W=128, k=0, q_rows=[128 * 3000 - 1],
         B=3, decode_tail=True),
    dict(dtype="bf16", H=128, D=128, T=4 * 20000, m=4, W=128, k=512, q_rows=[4 * 20000 - 1],
         B=2, decode_tail=True),
    dict(dtype="bf16", H=128, D=128, T=4 * 20000, m=4, W=128, k=0, q_rows=[4 * 20000 - 1],
         B=1, decode_tail=True),
    dict(dtype="bf16", H=128, D=64, T=4 * 7001, m=4, W=128, k=300, q_rows=[4 * 7001 - 3],
         B=3, decode_tail=True),
])
def test_decode_split(case):
    say("decode split", case)
    attend_case(**case)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_attend_wide_score_range(kind):
    """A key far above the first tile's scores (about 90 in the exp2 domain)
    in a later tile of every row: the running maximum must move by far more
    than the lazy rescaling threshold, with the split partials merged."""
    H, D, T, W = 128, 128, 3000, 128
    m = 4 if kind == "csa" else 16
    k = 64
    q_rows = rows(2900, 5)
    w = I.Workload("t", "csa", seed=57, dtype="bf16", B=1, T=T, m=m, H=H, D=D, W=W, k=k,
                   Tq=len(q_rows), q_pos0=q_rows[0])
    say("wide score range", kind)
    Nc = T // m
    q = torch.full((1, len(q_rows), H, D), 0.25, dtype=torch.bfloat16)
    ck = I.draw_cache(w, "ck", Nc)
    cv = I.draw_cache(w, "cv", Nc)
    rk = I.draw_cache(w, "rk", T)
    rv = I.draw_cache(w, "rv", T)
    q_pos = np.asarray(q_rows)
    if kind == "csa":
        rng = np.random.default_rng(5)
        tk = np.array([[random_selection(rng, oracle.n_cand(t, m, W), k) for t in q_pos]],
                      np.int32)
        for r in range(len(q_rows)):
            ck[0, int(tk[0, r, 45])] = 2.0          # kept-list position 45: the second tile
        ref = oracle.attend(f64(q), f64(ck), f64(cv), tk, f64(rk), f64(rv), 0, q_pos, m, W)
        got = csa.csa_attend(q.to(DEV), ck.to(DEV), cv.to(DEV), torch.from_numpy(tk).to(DEV),
                             rk.to(DEV), rv.to(DEV), m=m, W=W, q_pos0=int(q_pos[0]), raw_pos0=0)
    else:
        ck[0, 100] = 2.0                             # the fourth compressed tile
        ref = oracle.attend(f64(q), f64(ck), f64(cv), None, f64(rk), f64(rv), 0, q_pos, m, W)
        got = csa.hca_attend(q.to(DEV), ck.to(DEV), cv.to(DEV), rk.to(DEV), rv.to(DEV), m=m,
                             W=W, q_pos0=int(q_pos[0]), raw_pos0=0)
    torch.cuda.synchronize()
    err = maxerr(got, ref)
    say("  max err", err)
    assert err <= TOL["bf16"]


# ---------------------------------------------------------------- end to end
def test_tiny_config_end_to_end():
    """compress -> MXFP4 keys -> index/top-k -> attend on the tiny fp32 CSA
    workload, both sides from the same raw inputs."""
    w = I.TINY_CSA
    say("tiny end to end")
    raw = I.draw_raw(w)
    k_idx = I.draw_indexer_keys(w)
    q_idx = I.draw_indexer_queries(w)
    q = I.draw_queries(w)
    q_pos = np.arange(w.q_pos0, w.q_pos0 + w.Tq)
    # oracle chain
    ck = oracle.compress(f64(raw["k"]), f64(raw["gk"]), w.m)
    cv = oracle.compress(f64(raw["v"]), f64(raw["gv"]), w.m)
    kc, ks = oracle.quant_mxfp4(f64(k_idx))
    tk, exact = oracle.index_topk(f64(q_idx), kc, ks, q_pos, w.m, w.W, w.k)
    assert exact
    ref = oracle.attend(f64(q), ck, cv, tk, f64(raw["k"]), f64(raw["v"]), 0, q_pos, w.m, w.W)
    # GPU chain
    d = {n: t.to(DEV) for n, t in raw.items()}
    gck = csa.hca_compress(d["k"], d["gk"], w.m)
    gcv = csa.hca_compress(d["v"], d["gv"], w.m)
    gkc, gks = csa.csa_quantize_mxfp4(k_idx.to(DEV))
    gtk = csa.csa_index_topk(q_idx.to(DEV), gkc, gks, m=w.m, W=w.W, k=w.k, q_pos0=w.q_pos0)
    go = csa.csa_attend(q.to(DEV), gck, gcv, gtk, d["k"], d["v"], m=w.m, W=w.W,
                        q_pos0=w.q_pos0, raw_pos0=0)
    torch.cuda.synchronize()
    assert np.array_equal(gtk.cpu().numpy(), tk)
    err = maxerr(go, ref)
    say("  max err", err)
    assert err <= TOL["f32"]


def test_determinism_bitwise():
    """Two runs of the bf16 chain give identical bits (no atomics on values,
    fixed reduction orders)."""
    say("determinism")
    w = I.Workload("t", "csa", seed=41, dtype="bf16", B=1, T=9000, m=4, H=128, D=128, Tq=64,
                   q_pos0=8936)
    raw = {n: t.to(DEV) for n, t in I.draw_raw(w).items()}
    k_idx = I.draw_indexer_keys(w).to(DEV)
    q_idx = I.draw_indexer_queries(w).to(DEV)
    q = I.draw_queries(w).to(DEV)

    def run():
        ck = csa.hca_compress(raw["k"], raw["gk"], w.m)
        cv = csa.hca_compress(raw["v"], raw["gv"], w.m)
        kc, ks = csa.csa_quantize_mxfp4(k_idx)
        tk = csa.csa_index_topk(q_idx, kc, ks, m=w.m, W=w.W, k=w.k, q_pos0=w.q_pos0)
        o = csa.csa_attend(q, ck, cv, tk, raw["k"], raw["v"], m=w.m, W=w.W, q_pos0=w.q_pos0,
                           raw_pos0=0)
        torch.cuda.synchronize()
        return tk.cpu(), o.cpu()

    a, b = run(), run()
    assert torch.equal(a[0], b[0])
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_attend_wide_score_many_rows(kind):
    """Raw row 2700 far above the other keys (about 90 in the exp2 domain):
    the 128 rows whose window holds it meet it in a later tile than the
    first, so their running maximum must move by far more than the lazy
    rescaling threshold; the other rows of the launch never see it."""
    H, D, T, W = 128, 128, 3000, 128
    m = 4 if kind == "csa" else 16
    k = 64
    q_rows = rows(2400, 600)
    w = I.Workload("t", "csa", seed=58, dtype="bf16", B=1, T=T, m=m, H=H, D=D, W=W, k=k,
                   Tq=len(q_rows), q_pos0=q_rows[0])
    say("wide score range, many rows", kind)
    Nc = T // m
    q = torch.full((1, len(q_rows), H, D), 0.25, dtype=torch.bfloat16)
    ck = I.draw_cache(w, "ck", Nc)
    cv = I.draw_cache(w, "cv", Nc)
    rk = I.draw_cache(w, "rk", T)
    rv = I.draw_cache(w, "rv", T)
    rk[0, 2700] = 2.0
    q_pos = np.asarray(q_rows)
    if kind == "csa":
        rng = np.random.default_rng(6)
        tk = np.array([[random_selection(rng, oracle.n_cand(t, m, W), k) for t in q_pos]],
                      np.int32)
        ref = oracle.attend(f64(q), f64(ck), f64(cv), tk, f64(rk), f64(rv), 0, q_pos, m, W)
        got = csa.csa_attend(q.to(DEV), ck.to(DEV), cv.to(DEV), torch.from_numpy(tk).to(DEV),
                             rk.to(DEV), rv.to(DEV), m=m, W=W, q_pos0=int(q_pos[0]), raw_pos0=0)
    else:
        ref = oracle.attend(f64(q), f64(ck), f64(cv), None, f64(rk), f64(rv), 0, q_pos, m, W)
        got = csa.hca_attend(q.to(DEV), ck.to(DEV), cv.to(DEV), rk.to(DEV), rv.to(DEV), m=m,
                             W=W, q_pos0=int(q_pos[0]), raw_pos0=0)
    torch.cuda.synchronize()
    err = maxerr(got, ref)
    say("  max err", err)
    assert err <= TOL["bf16"]
