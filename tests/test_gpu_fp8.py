"""FP8 attention arithmetic on the GPU against the oracle (reading R13d;
ai-papers.net article, hybrid attention section: most KV entries in FP8).

* csa_quantize_fp8_rows is bit-exact against the oracle's row encoding.
* csa_attend_fp8 / hca_attend_fp8 take FP8 rows (entries and window, encoded
  by the oracle) and bf16 queries, and are compared with the oracle's
  attend_fp8 (queries encoded per head row, exact attention over the decoded
  rows).  The kernel rounds each probability, times its value row's
  exponent, to E4M3 for the value product: a relative error of at most 2^-4
  per probability, so every output element obeys
      |o_gpu - o| <= 2^-4 * amean + 2^-8 |o| + 3e-3
  (amean = sum p|v| / sum p from the oracle; the last two terms cover the
  bf16 output and split records, fp32 sums and probabilities in the E4M3
  subnormal range), and the mean of ((o_gpu - o) / rms)^2 over the elements
  (rms = sqrt(sum p^2 v^2) / sum p) stays below (0.6 * 2^-4)^2, about twice
  what independent roundings give (0.18 * 2^-8): a systematic error of a
  few percent in any weight or value fails it."""
import numpy as np
import pytest
import torch

import oracle
from compressed_sparse_attention_04_amd import binding as csa
from compressed_sparse_attention_04_amd import inputs as I
from tests.gpu_helpers import DEV, check_fp8 as check, f64, fp8_host_rows as host_rows, \
    random_selection, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,rows,d,kind", [
    ("bf16", 1000, 128, "normal"),
    ("f32", 333, 64, "normal"),
    ("f32", 64, 32, "ties"),
    ("bf16", 50, 256, "wide"),
    ("f32", 40, 128, "edge"),
    ("bf16", 7, 128, "normal"),
])
def test_quantize_rows_bit_exact(dtype, rows, d, kind):
    say("quantize_fp8_rows", dtype, rows, d, kind)
    g = torch.Generator().manual_seed(rows + d + 1)
    x = torch.randn(rows, d, generator=g, dtype=torch.float64)
    if kind == "ties":
        mids = torch.tensor([1.0625, 1.1875, 17.0, 19.0, 1.5 * 2 ** -9, 0.5 * 2 ** -9, 2.5 * 2 ** -9,
                             -3.25 * 2 ** -3, 460.0, 240.0], dtype=torch.float64)
        x = mids[torch.randint(0, len(mids), (rows, d), generator=g)]
        x[:, 0] = 300.0
    elif kind == "wide":
        x = x * torch.exp2(torch.randint(-60, 60, (rows, 1), generator=g).double())
        x[:, 5:40] *= 2.0 ** -20                         # runs far below the row maximum
    elif kind == "edge":
        x[0:10] = 0.0                                    # zero rows
        x[10:20, :16] = -0.0
        x[20:30] *= 2.0 ** -140                          # subnormal fp32 maxima
        x[30:40] *= 2.0 ** 100
    xt = x.to(I.torch_dtype(dtype))
    codes, scales = csa.csa_quantize_fp8_rows(xt.to(DEV))
    torch.cuda.synchronize()
    rc, rs = oracle.quant_fp8_rows(f64(xt))
    # one scale word per row: the fp32 bits of 2^e, the oracle's byte e + 127
    # in bits 23..30 (the oracle repeats that byte in each 32-value slot)
    assert np.array_equal(scales.cpu().numpy(), rs[:, 0].astype(np.int32) << 23)
    assert np.array_equal(codes.cpu().numpy(), rc)


def enc(t):
    """The oracle's FP8 rows of t; on the device as codes and one scale word
    per row (the row's exponent byte in bits 23..30)."""
    c, s = oracle.quant_fp8_rows(f64(t))
    return torch.from_numpy(c).to(DEV), torch.from_numpy(s[..., 0].astype(np.int32) << 23).to(DEV)


def fp8_case(H, T, m, W, k, q_rows, B=1, seed=51, decode_tail=False, corrupt=False,
             wide=False):
    w = I.Workload("t", "csa", seed=seed, dtype="bf16", B=B, T=T, m=m, H=H, D=128, W=W,
                   k=max(k, 1), Tq=len(q_rows), q_pos0=int(q_rows[0]))
    Nc = T // m
    q = I.draw_queries(w)
    ck = I.draw_cache(w, "ck", Nc)
    cv = I.draw_cache(w, "cv", Nc)
    if wide:
        # value rows whose exponents spread over 8 octaves and key rows over 4
        # (P stays in E4M3's normal range while p * 2^(e_v - E) >= 2^-12, E
        # the largest value exponent of the 64 keys processed together)
        g = torch.Generator().manual_seed(seed)
        cv = (cv.double() * torch.exp2(torch.randint(-4, 5, (B, Nc, 1), generator=g).double())
              ).to(cv.dtype)
        ck = (ck.double() * torch.exp2(torch.randint(-2, 3, (B, Nc, 1), generator=g).double())
              ).to(ck.dtype)
    if decode_tail:
        raw_pos0 = int(q_rows[0]) - W + 1
        rk, rv = I.draw_cache(w, "rk", W), I.draw_cache(w, "rv", W)
    else:
        raw_pos0 = 0
        rk, rv = I.draw_cache(w, "rk", T), I.draw_cache(w, "rv", T)
    # the oracle encodes every row; both sides read these codes
    (kc, ks), (vc, vs), (rkc, rks), (rvc, rvs) = enc(ck), enc(cv), enc(rk), enc(rv)
    host = [a for pair in ((kc, ks), (vc, vs), (rkc, rks), (rvc, rvs)) for a in host_rows(*pair)]
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
        ref = oracle.attend_fp8(f64(q), *host[:4], tk, *host[4:], raw_pos0, q_pos, m, W)
        got = csa.csa_attend_fp8(q.to(DEV), kc, vc, ks, vs, torch.from_numpy(tk).to(DEV), rkc, rvc,
                                 rks, rvs, m=m, W=W, q_pos0=int(q_pos[0]), raw_pos0=raw_pos0)
    else:
        ref = oracle.attend_fp8(f64(q), *host[:4], None, *host[4:], raw_pos0, q_pos, m, W)
        got = csa.hca_attend_fp8(q.to(DEV), kc, vc, ks, vs, rkc, rvc, rks, rvs, m=m, W=W,
                                 q_pos0=int(q_pos[0]), raw_pos0=raw_pos0)
    torch.cuda.synchronize()
    check(got, ref)


def rows(a, n):
    return list(range(a, a + n))


@pytest.mark.parametrize("case", [
    dict(H=128, T=3000, m=4, W=128, k=64, q_rows=rows(2900, 33)),
    dict(H=128, T=6000, m=4, W=128, k=512, q_rows=rows(5500, 9), B=2),       # splits
    dict(H=32, T=2000, m=4, W=40, k=100, q_rows=rows(1000, 17)),
    dict(H=64, T=2500, m=4, W=100, k=200, q_rows=rows(1, 51)),               # early rows
    dict(H=256, T=2000, m=4, W=128, k=32, q_rows=rows(1900, 3)),
    dict(H=128, T=4000, m=4, W=128, k=512, q_rows=rows(3000, 20), corrupt=True),
    dict(H=128, T=4000, m=4, W=128, k=512, q_rows=rows(3000, 20), wide=True),
    dict(H=128, T=3000, m=4, W=128, k=64, q_rows=rows(2000, 600)),           # no splits
    dict(H=128, T=40000, m=4, W=128, k=512, q_rows=[39999], B=3, decode_tail=True),
])
def test_csa_attend_fp8(case):
    say("csa_attend_fp8", case)
    fp8_case(**case)


@pytest.mark.parametrize("case", [
    dict(H=128, T=5000, m=128, W=128, k=0, q_rows=rows(4950, 40)),
    dict(H=128, T=700, m=4, W=64, k=0, q_rows=rows(0, 30)),
    dict(H=64, T=3000, m=16, W=128, k=0, q_rows=rows(2000, 37)),
    dict(H=128, T=40000, m=128, W=128, k=0, q_rows=[39999], B=4, decode_tail=True),
    dict(H=128, T=40000, m=128, W=128, k=0, q_rows=[39999], B=2, decode_tail=True, wide=True),
    dict(H=128, T=20000, m=128, W=128, k=0, q_rows=rows(19000, 520)),
    dict(H=32, T=9000, m=4, W=128, k=0, q_rows=rows(8990, 3)),
])
def test_hca_attend_fp8(case):
    say("hca_attend_fp8", case)
    fp8_case(**case)


def test_fp8_rows_from_the_library_encoder():
    """The library's own encoder feeding the attention gives the oracle's codes."""
    case = dict(H=128, T=40000, m=128, W=128, k=0, q_rows=[39999], B=2, decode_tail=True)
    w = I.Workload("t", "csa", seed=7, dtype="bf16", B=2, T=40000, m=128, H=128, D=128, W=128,
                   k=1, Tq=1, q_pos0=39999)
    cv = I.draw_cache(w, "cv", 312)
    c1, s1 = csa.csa_quantize_fp8_rows(cv.to(DEV))
    c2, s2 = enc(cv)
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    fp8_case(**case)
