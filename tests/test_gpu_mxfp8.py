"""Compressed entries stored as MXFP8 (ai-papers.net article, hybrid
attention section: most KV entries in FP8) on the GPU against the oracle.

* csa_quantize_mxfp8 is bit-exact against the oracle's encoding.
* csa_attend_mxfp8 / hca_attend_mxfp8 take the oracle's codes and scales
  and match the oracle's attention over the exactly decoded entries (window
  rows in bf16) within the bf16 bar, on ragged, split (decode), shared-vector,
  corrupted-list and many-row launches."""
import numpy as np
import pytest
import torch

import oracle
from compressed_sparse_attention_04_amd import binding as csa
from compressed_sparse_attention_04_amd import inputs as I
from tests.gpu_helpers import DEV, TOL, f64, maxerr, random_selection, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,rows,d,kind", [
    ("bf16", 1000, 128, "normal"),
    ("f32", 333, 64, "normal"),
    ("f32", 64, 32, "ties"),
    ("bf16", 50, 256, "wide"),
    ("f32", 40, 128, "edge"),
])
def test_quantize_bit_exact(dtype, rows, d, kind):
    say("quantize_mxfp8", dtype, rows, d, kind)
    g = torch.Generator().manual_seed(rows + d)
    x = torch.randn(rows, d, generator=g, dtype=torch.float64)
    if kind == "ties":
        # blocks scaled by 2^0 whose other values sit exactly on E4M3 midpoints
        mids = torch.tensor([1.0625, 1.1875, 17.0, 19.0, 1.5 * 2 ** -9, 0.5 * 2 ** -9, 2.5 * 2 ** -9,
                             -3.25 * 2 ** -3, 460.0, 240.0], dtype=torch.float64)
        x = mids[torch.randint(0, len(mids), (rows, d), generator=g)]
        x[:, ::32] = 300.0
    elif kind == "wide":
        x = x * torch.exp2(torch.randint(-60, 60, (rows, 1), generator=g).double())
    elif kind == "edge":
        x[0:10] = 0.0                                    # all-zero runs
        x[10:20, :16] = -0.0
        x[20:30] *= 2.0 ** -140                          # subnormal fp32 maxima
        x[30:40] *= 2.0 ** 100
    xt = x.to(I.torch_dtype(dtype))
    codes, scales = csa.csa_quantize_mxfp8(xt.to(DEV))
    torch.cuda.synchronize()
    rc, rs = oracle.quant_mxfp8(f64(xt))
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def mx8_case(H, T, m, W, k, q_rows, B=1, seed=41, decode_tail=False, corrupt=False,
             shared=False):
    w = I.Workload("t", "csa", seed=seed, dtype="bf16", B=B, T=T, m=m, H=H, D=128, W=W,
                   k=max(k, 1), Tq=len(q_rows), q_pos0=int(q_rows[0]))
    Nc = T // m
    q = I.draw_queries(w)
    ck = I.draw_cache(w, "ck", Nc)
    cv = ck if shared else I.draw_cache(w, "cv", Nc)
    if decode_tail:
        raw_pos0 = int(q_rows[0]) - W + 1
        rk = I.draw_cache(w, "rk", W)
        rv = rk if shared else I.draw_cache(w, "rv", W)
    else:
        raw_pos0 = 0
        rk = I.draw_cache(w, "rk", T)
        rv = rk if shared else I.draw_cache(w, "rv", T)
    # the oracle encodes the entries; both sides read these codes
    kc, ks = oracle.quant_mxfp8(f64(ck))
    vc, vs = (kc, ks) if shared else oracle.quant_mxfp8(f64(cv))
    ck_dq, cv_dq = oracle.dequant_mxfp8(kc, ks), oracle.dequant_mxfp8(vc, vs)
    d_kc, d_ks = torch.from_numpy(kc).to(DEV), torch.from_numpy(ks).to(DEV)
    d_vc, d_vs = (d_kc, d_ks) if shared else (torch.from_numpy(vc).to(DEV),
                                               torch.from_numpy(vs).to(DEV))
    d_rk = rk.to(DEV)
    d_rv = d_rk if shared else rv.to(DEV)
    q_pos = np.asarray(q_rows)
    rng = np.random.default_rng(seed)
    if k > 0:
        tk = np.array([[random_selection(rng, oracle.n_cand(t, m, W), k) for t in q_pos]
                       for _ in range(B)], np.int32)
        if corrupt:
            nc = np.array([oracle.n_cand(t, m, W) for t in q_pos])
            bad = rng.random(tk.shape) < 0.125
            junk = np.where(rng.random(tk.shape) < 0.5, -1, nc[None, :, None] + 3)
            tk = np.where(bad, junk, tk).astype(np.int32)
        ref = oracle.attend(f64(q), ck_dq, cv_dq, tk, f64(rk), f64(rv), raw_pos0, q_pos, m, W)
        got = csa.csa_attend_mxfp8(q.to(DEV), d_kc, d_vc, d_ks, d_vs,
                                   torch.from_numpy(tk).to(DEV), d_rk, d_rv, m=m, W=W,
                                   q_pos0=int(q_pos[0]), raw_pos0=raw_pos0)
    else:
        ref = oracle.attend(f64(q), ck_dq, cv_dq, None, f64(rk), f64(rv), raw_pos0, q_pos, m, W)
        got = csa.hca_attend_mxfp8(q.to(DEV), d_kc, d_vc, d_ks, d_vs, d_rk, d_rv, m=m, W=W,
                                   q_pos0=int(q_pos[0]), raw_pos0=raw_pos0)
    torch.cuda.synchronize()
    err = maxerr(got, ref)
    say("  max err", err)
    assert err <= TOL["bf16"]


def rows(a, n):
    return list(range(a, a + n))


@pytest.mark.parametrize("case", [
    dict(H=128, T=3000, m=4, W=128, k=64, q_rows=rows(2900, 33)),
    dict(H=128, T=6000, m=4, W=128, k=512, q_rows=rows(5500, 9), B=2),       # splits
    dict(H=32, T=2000, m=4, W=40, k=100, q_rows=rows(1000, 17)),
    dict(H=64, T=2500, m=4, W=100, k=200, q_rows=rows(1, 51)),               # early rows
    dict(H=256, T=2000, m=4, W=128, k=32, q_rows=rows(1900, 3)),
    dict(H=128, T=4000, m=4, W=128, k=512, q_rows=rows(3000, 20), corrupt=True),
    dict(H=128, T=4000, m=4, W=128, k=512, q_rows=rows(3000, 20), shared=True),
    dict(H=128, T=3000, m=4, W=128, k=64, q_rows=rows(2000, 600)),           # no splits
    dict(H=128, T=40000, m=4, W=128, k=512, q_rows=[39999], B=3, decode_tail=True),
])
def test_csa_attend_mxfp8(case):
    say("csa_attend_mxfp8", case)
    mx8_case(**case)


@pytest.mark.parametrize("case", [
    dict(H=128, T=5000, m=128, W=128, k=0, q_rows=rows(4950, 40)),
    dict(H=128, T=700, m=4, W=64, k=0, q_rows=rows(0, 30)),
    dict(H=64, T=3000, m=16, W=128, k=0, q_rows=rows(2000, 37)),
    dict(H=128, T=40000, m=128, W=128, k=0, q_rows=[39999], B=4, decode_tail=True),
    dict(H=128, T=40000, m=128, W=128, k=0, q_rows=[39999], B=2, decode_tail=True,
         shared=True),
    dict(H=128, T=20000, m=128, W=128, k=0, q_rows=rows(19000, 520)),
])
def test_hca_attend_mxfp8(case):
    say("hca_attend_mxfp8", case)
    mx8_case(**case)
