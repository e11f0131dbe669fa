"""Parity at the full sizes of the benchmarked workloads, in the launch
configuration bench.py times (same entry points, shapes, workspaces and
paths), checked against the oracle on sampled outputs it can compute one by
one: sampled query rows (prefill) or sampled sequences (decode).  The MXFP8
cases run bench.py --kv-format mxfp8's chain (pooling, encoding, MXFP8
attention) against the oracle's pooling, encoding and attention over the
decoded entries.

The inputs are drawn on the GPU by the shared input module and copied to the
host for the oracle, so both sides see the same numbers.  The oracle runs its
own chain from the raw inputs (its own compression, MXFP4 encoding, scores
and top-k) and never takes an intermediate result of the GPU path, with one
exception: the FP8 decode cases (bench.py --kv-format fp8) check the GPU's
pooled caches against the oracle's pooling, then hand those bf16 caches to
the oracle's FP8 row encoder, whose codes must equal the library's bit for
bit, so that the FP8 attention on both sides reads the same codes (an E4M3
code can flip where the two poolings round differently, which the FP8
attention bound does not cover).
"""
import numpy as np
import pytest
import torch

import oracle
from compressed_sparse_attention_04_amd import binding as csa
from compressed_sparse_attention_04_amd import inputs as I
from tests.gpu_helpers import DEV, TOL, check_fp8, f64, fp8_host_rows, maxerr, say

pytestmark = pytest.mark.gpu


def sample_rows(w, fixed, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set(r for r in fixed if 0 <= r < w.Tq)
    rows |= set(rng.choice(w.Tq, size=n_random, replace=False).tolist())
    return np.array(sorted(rows), np.int64)


def prefill_layer(w, rows, kv_fmt="bf16"):
    """Full GPU chain of one prefill layer, then the oracle's chain for the
    sampled query rows.  kv_fmt "mxfp8": the compressed entries are encoded
    to MXFP8 after pooling and attention reads them so (bench.py
    --kv-format mxfp8); the oracle encodes its own pooled entries."""
    say("full size", w.name, kv_fmt, "rows", rows.tolist())
    raw = I.draw_raw(w, device=DEV)
    gck = csa.hca_compress(raw["k"], raw["gk"], w.m)
    gcv = csa.hca_compress(raw["v"], raw["gv"], w.m)
    q = I.draw_queries(w, device=DEV)
    if w.kind == "csa":
        k_idx = I.draw_indexer_keys(w, device=DEV)
        gkc, gks = csa.csa_quantize_mxfp4(k_idx)
        q_idx = I.draw_indexer_queries(w, device=DEV)
        ws = torch.empty(max(1, csa.csa_index_topk_workspace(w.B, w.Tq, w.HI, w.dI, w.Nc, w.m,
                                                               w.W, w.k, w.q_pos0)),
                         dtype=torch.uint8, device=DEV)
        gtk = csa.csa_index_topk(q_idx, gkc, gks, m=w.m, W=w.W, k=w.k, q_pos0=w.q_pos0, ws=ws)
        del q_idx, ws
    if kv_fmt == "mxfp8":
        (kc8, ks8), (vc8, vs8) = csa.csa_quantize_mxfp8(gck), csa.csa_quantize_mxfp8(gcv)
        if w.kind == "csa":
            go = csa.csa_attend_mxfp8(q, kc8, vc8, ks8, vs8, gtk, raw["k"], raw["v"], m=w.m,
                                      W=w.W, q_pos0=w.q_pos0, raw_pos0=0)
        else:
            go = csa.hca_attend_mxfp8(q, kc8, vc8, ks8, vs8, raw["k"], raw["v"], m=w.m, W=w.W,
                                      q_pos0=w.q_pos0, raw_pos0=0)
    elif w.kind == "csa":
        go = csa.csa_attend(q, gck, gcv, gtk, raw["k"], raw["v"], m=w.m, W=w.W,
                            q_pos0=w.q_pos0, raw_pos0=0)
    else:
        go = csa.hca_attend(q, gck, gcv, raw["k"], raw["v"], m=w.m, W=w.W, q_pos0=w.q_pos0,
                            raw_pos0=0)
    torch.cuda.synchronize()
    del q
    sel = torch.from_numpy(rows).to(DEV)
    got = go[:, sel].cpu()
    del go
    host = {n: f64(t.cpu()) for n, t in raw.items()}
    # oracle chain
    ck = oracle.compress(host["k"], host["gk"], w.m)
    cv = oracle.compress(host["v"], host["gv"], w.m)
    err_c = max(maxerr(gck.cpu(), ck), maxerr(gcv.cpu(), cv))
    say("  compressed caches max err", err_c)
    assert err_c <= TOL[w.dtype]
    if kv_fmt == "mxfp8":
        ck, cv = oracle.dequant_mxfp8(*oracle.quant_mxfp8(ck)), oracle.dequant_mxfp8(
            *oracle.quant_mxfp8(cv))
    q_pos = w.q_pos0 + rows
    qh = f64(I.draw_queries(w, device=DEV, rows=rows).cpu())
    if w.kind == "csa":
        kc, ks = oracle.quant_mxfp4(f64(k_idx.cpu()))
        assert np.array_equal(gkc.cpu().numpy(), kc) and np.array_equal(gks.cpu().numpy(), ks)
        qi = f64(I.draw_indexer_queries(w, device=DEV, rows=rows).cpu())
        tk, exact = oracle.index_topk(qi, kc, ks, q_pos, w.m, w.W, w.k)
        assert exact
        g_tk = gtk[:, sel].cpu().numpy()
        bad = np.argwhere((g_tk != tk).any(axis=2))
        assert bad.size == 0, f"index rows differ: {rows[bad[:, 1]].tolist()}"
        ref = oracle.attend(qh, ck, cv, tk, host["k"], host["v"], 0, q_pos, w.m, w.W)
    else:
        ref = oracle.attend(qh, ck, cv, None, host["k"], host["v"], 0, q_pos, w.m, w.W)
    err = maxerr(got, ref)
    say("  output max err", err)
    assert err <= TOL[w.dtype]


def test_csa_prefill_32k_full_size():
    w = I.CSA_PREFILL_32K
    rows = sample_rows(w, [0, 1, 127, 128, 129, 2174, 2175, 2176, 2177, 4095, 4096, 16383,
                           32766, 32767], 8, seed=101)
    prefill_layer(w, rows)


@pytest.mark.parametrize("w", [I.PAIR_CSA_128K, I.PAIR_HCA_128K], ids=lambda w: w.name)
def test_pair_prefill_128k_full_size(w):
    fixed = [0, 126, 127, 128, 255, 256, 2175, 2176, 8191, 8192, 65535, 65536, 131070, 131071]
    prefill_layer(w, sample_rows(w, fixed, 6, seed=102))


@pytest.mark.parametrize("w", [I.PAIR_CSA_128K, I.PAIR_HCA_128K], ids=lambda w: w.name)
def test_pair_prefill_128k_full_size_mxfp8(w):
    fixed = [0, 127, 128, 2176, 65536, 131071]
    prefill_layer(w, sample_rows(w, fixed, 4, seed=103), kv_fmt="mxfp8")


def decode_caches_gpu(w, with_keys):
    """Per-sequence chunked compression of the whole context on the GPU, the
    last W raw rows kept (the decode workload's precompressed caches)."""
    L = I.chunk_len(w)
    per = L // w.m
    ck = torch.empty((w.B, w.Nc, w.D), dtype=torch.bfloat16, device=DEV)
    cv = torch.empty_like(ck)
    rk = torch.empty((w.B, w.W, w.D), dtype=torch.bfloat16, device=DEV)
    rv = torch.empty_like(rk)
    nchunks = w.T // L
    for b in range(w.B):
        for c in range(nchunks):
            x = {n: I.draw_chunk(w, n, b, c, device=DEV)[None] for n in ("k", "v", "gk", "gv")}
            csa.hca_compress(x["k"], x["gk"], w.m, out=ck[b:b + 1, c * per:(c + 1) * per])
            csa.hca_compress(x["v"], x["gv"], w.m, out=cv[b:b + 1, c * per:(c + 1) * per])
            if c == nchunks - 1:
                rk[b].copy_(x["k"][0, -w.W:])
                rv[b].copy_(x["v"][0, -w.W:])
    return ck, cv, rk, rv


def decode_caches_oracle(w, b):
    """The oracle's own compression of sequence b, chunk by chunk."""
    L = I.chunk_len(w)
    ck, cv = [], []
    for c in range(w.T // L):
        x = {n: f64(I.draw_chunk(w, n, b, c, device=DEV).cpu())[None]
             for n in ("k", "v", "gk", "gv")}
        ck.append(oracle.compress(x["k"], x["gk"], w.m)[0])
        cv.append(oracle.compress(x["v"], x["gv"], w.m)[0])
        if c == w.T // L - 1:
            rk, rv = x["k"][0, -w.W:], x["v"][0, -w.W:]
    return np.concatenate(ck)[None], np.concatenate(cv)[None], rk[None], rv[None]


@pytest.mark.parametrize("name,seqs,kv_fmt", [("hca_decode_1m", [0, 31], "bf16"),
                                              ("csa_decode_1m", [9], "bf16"),
                                              ("hca_decode_1m", [5], "mxfp8"),
                                              ("csa_decode_1m", [14], "mxfp8")])
def test_decode_1m_full_size(name, seqs, kv_fmt):
    w = I.HCA_DECODE_1M if name == "hca_decode_1m" else I.CSA_DECODE_1M
    t = w.q_pos0
    say("full size", w.name, kv_fmt, "sequences", seqs)
    ck, cv, rk, rv = decode_caches_gpu(w, w.kind == "csa")
    if kv_fmt == "mxfp8":
        mx = csa.csa_quantize_mxfp8(ck) + csa.csa_quantize_mxfp8(cv)   # kc, ks, vc, vs
    q = I.draw_queries(w, device=DEV)
    if w.kind == "csa":
        k_idx = I.draw_indexer_keys(w, device=DEV)
        gkc, gks = csa.csa_quantize_mxfp4(k_idx)
        q_idx = I.draw_indexer_queries(w, device=DEV)
        iws = torch.empty(max(1, csa.csa_index_topk_workspace(w.B, 1, w.HI, w.dI, w.Nc, w.m, w.W,
                                                                w.k, t)),
                          dtype=torch.uint8, device=DEV)
        aws = torch.empty(max(1, csa.csa_attend_workspace(1, w.B, 1, w.H, w.D, w.k, w.W)),
                          dtype=torch.uint8, device=DEV)
        gtk = csa.csa_index_topk(q_idx, gkc, gks, m=w.m, W=w.W, k=w.k, q_pos0=t, ws=iws)
        if kv_fmt == "mxfp8":
            go = csa.csa_attend_mxfp8(q, mx[0], mx[2], mx[1], mx[3], gtk, rk, rv, m=w.m, W=w.W,
                                      q_pos0=t, raw_pos0=t - w.W + 1, ws=aws)
        else:
            go = csa.csa_attend(q, ck, cv, gtk, rk, rv, m=w.m, W=w.W, q_pos0=t,
                                raw_pos0=t - w.W + 1, ws=aws)
    else:
        aws = torch.empty(max(1, csa.hca_attend_workspace(1, w.B, 1, w.H, w.D, w.Nc, w.m, w.W,
                                                          t)), dtype=torch.uint8, device=DEV)
        if kv_fmt == "mxfp8":
            go = csa.hca_attend_mxfp8(q, mx[0], mx[2], mx[1], mx[3], rk, rv, m=w.m, W=w.W,
                                      q_pos0=t, raw_pos0=t - w.W + 1, ws=aws)
        else:
            go = csa.hca_attend(q, ck, cv, rk, rv, m=w.m, W=w.W, q_pos0=t, raw_pos0=t - w.W + 1,
                                ws=aws)
    torch.cuda.synchronize()
    for b in seqs:
        ock, ocv, ork, orv = decode_caches_oracle(w, b)
        err_c = max(maxerr(ck[b:b + 1].cpu(), ock), maxerr(cv[b:b + 1].cpu(), ocv))
        say("  sequence", b, "compressed caches max err", err_c)
        assert err_c <= TOL[w.dtype]
        qh = f64(q[b:b + 1].cpu())
        if w.kind == "csa":
            kc, ks = oracle.quant_mxfp4(f64(k_idx[b:b + 1].cpu()))
            tk, exact = oracle.index_topk(f64(q_idx[b:b + 1].cpu()), kc, ks, [t], w.m, w.W, w.k)
            assert exact
            assert np.array_equal(gtk[b:b + 1].cpu().numpy(), tk)
        else:
            tk = None
        if kv_fmt == "mxfp8":
            ock = oracle.dequant_mxfp8(*oracle.quant_mxfp8(ock))
            ocv = oracle.dequant_mxfp8(*oracle.quant_mxfp8(ocv))
        ref = oracle.attend(qh, ock, ocv, tk, ork, orv, t - w.W + 1, [t], w.m, w.W)
        err = maxerr(go[b:b + 1].cpu(), ref)
        say("  sequence", b, "output max err", err)
        assert err <= TOL[w.dtype]


@pytest.mark.parametrize("name,seqs", [("hca_decode_1m", [3]), ("csa_decode_1m", [11])])
def test_decode_1m_full_size_fp8(name, seqs):
    """bench.py --kv-format fp8's decode step at full size: every entry and
    window row encoded to an FP8 row by the library, FP8 attention."""
    w = I.HCA_DECODE_1M if name == "hca_decode_1m" else I.CSA_DECODE_1M
    t = w.q_pos0
    say("full size", w.name, "fp8", "sequences", seqs)
    ck, cv, rk, rv = decode_caches_gpu(w, w.kind == "csa")
    f8 = {n: csa.csa_quantize_fp8_rows(x) for n, x in (("ck", ck), ("cv", cv), ("rk", rk),
                                                         ("rv", rv))}
    q = I.draw_queries(w, device=DEV)
    if w.kind == "csa":
        k_idx = I.draw_indexer_keys(w, device=DEV)
        gkc, gks = csa.csa_quantize_mxfp4(k_idx)
        q_idx = I.draw_indexer_queries(w, device=DEV)
        iws = torch.empty(max(1, csa.csa_index_topk_workspace(w.B, 1, w.HI, w.dI, w.Nc, w.m, w.W,
                                                                w.k, t)),
                          dtype=torch.uint8, device=DEV)
        aws = torch.empty(max(1, csa.csa_attend_workspace(1, w.B, 1, w.H, w.D, w.k, w.W)),
                          dtype=torch.uint8, device=DEV)
        gtk = csa.csa_index_topk(q_idx, gkc, gks, m=w.m, W=w.W, k=w.k, q_pos0=t, ws=iws)
        go = csa.csa_attend_fp8(q, f8["ck"][0], f8["cv"][0], f8["ck"][1], f8["cv"][1], gtk,
                                f8["rk"][0], f8["rv"][0], f8["rk"][1], f8["rv"][1], m=w.m, W=w.W,
                                q_pos0=t, raw_pos0=t - w.W + 1, ws=aws)
    else:
        aws = torch.empty(max(1, csa.hca_attend_workspace(1, w.B, 1, w.H, w.D, w.Nc, w.m, w.W,
                                                          t)), dtype=torch.uint8, device=DEV)
        go = csa.hca_attend_fp8(q, f8["ck"][0], f8["cv"][0], f8["ck"][1], f8["cv"][1],
                                f8["rk"][0], f8["rv"][0], f8["rk"][1], f8["rv"][1], m=w.m, W=w.W,
                                q_pos0=t, raw_pos0=t - w.W + 1, ws=aws)
    torch.cuda.synchronize()
    for b in seqs:
        ock, ocv, _, _ = decode_caches_oracle(w, b)
        err_c = max(maxerr(ck[b:b + 1].cpu(), ock), maxerr(cv[b:b + 1].cpu(), ocv))
        say("  sequence", b, "compressed caches max err", err_c)
        assert err_c <= TOL[w.dtype]
        host = {}
        for n, x in (("ck", ck), ("cv", cv), ("rk", rk), ("rv", rv)):
            oc, os_ = oracle.quant_fp8_rows(f64(x[b:b + 1].cpu()))
            gc, gs = fp8_host_rows(f8[n][0][b:b + 1], f8[n][1][b:b + 1])
            assert np.array_equal(gc, oc) and np.array_equal(gs, os_), n
            host[n] = (oc, os_)
        if w.kind == "csa":
            kc, ks = oracle.quant_mxfp4(f64(k_idx[b:b + 1].cpu()))
            tk, exact = oracle.index_topk(f64(q_idx[b:b + 1].cpu()), kc, ks, [t], w.m, w.W, w.k)
            assert exact
            assert np.array_equal(gtk[b:b + 1].cpu().numpy(), tk)
        else:
            tk = None
        ref = oracle.attend_fp8(f64(q[b:b + 1].cpu()), *host["ck"], *host["cv"], tk,
                                *host["rk"], *host["rv"], t - w.W + 1, [t], w.m, w.W)
        say("  sequence", b)
        check_fp8(go[b:b + 1].cpu(), ref)
