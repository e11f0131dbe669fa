"""Incremental decode append (hca_append) on the GPU against the oracle.

Tokens are appended one at a time.  Pinned three ways:
  * the compressed entries are bit-identical to a pooling of the whole
    sequence by hca_compress (same arithmetic);
  * they are within the dtype's bar of the oracle's pooling;
  * the window buffer holds exactly the newest raw rows.
A decode loop (append, index, attend per token) is checked against the
oracle's attention over the whole sequence's caches at every step."""
import numpy as np
import pytest
import torch

import oracle
from compressed_sparse_attention_04_amd import binding as csa
from compressed_sparse_attention_04_amd import inputs as I
from tests.gpu_helpers import DEV, TOL, f64, maxerr, say

pytestmark = pytest.mark.gpu


def new_state(w, C, gc, wcap, nc_cap, shared):
    dt = I.torch_dtype(w.dtype)
    z = lambda *s: torch.zeros(s, dtype=dt, device=DEV)
    st = {"rk": z(w.B, wcap, C), "gk": z(w.B, w.m, gc), "ck": z(w.B, nc_cap, C)}
    if shared:
        st.update(rv=st["rk"], gv=st["gk"], cv=st["ck"])
    else:
        st.update(rv=z(w.B, wcap, C), gv=z(w.B, w.m, gc), cv=z(w.B, nc_cap, C))
    return st


def append_range(st, raw, w, t0, t1, p0, shared):
    """Append positions t0 .. t1 - 1; returns the window's first position."""
    for t in range(t0, t1):
        kn = raw["k"][:, t].contiguous()
        gk = raw["gk"][:, t].contiguous()
        vn = kn if shared else raw["v"][:, t].contiguous()
        gv = gk if shared else raw["gv"][:, t].contiguous()
        p0 = csa.hca_append(kn, vn, gk, gv, st["rk"], st["rv"], st["gk"], st["gv"], st["ck"],
                            st["cv"], m=w.m, W=w.W, t=t, win_pos0=p0)
    return p0


@pytest.mark.parametrize("dtype,C,m,W,T,B,gate,shared", [
    ("bf16", 128, 4, 128, 600, 2, "channel", False),
    ("bf16", 128, 128, 128, 700, 1, "channel", False),    # m = W: blocks fill the window
    ("f32", 64, 4, 32, 300, 1, "token", False),
    ("bf16", 64, 17, 40, 400, 3, "channel", False),       # m > 16: row groups, ragged tail
    ("bf16", 128, 16, 128, 500, 1, "token", False),
    ("bf16", 128, 1, 16, 100, 1, "channel", False),       # m = 1: every token an entry
    ("bf16", 128, 4, 128, 400, 2, "channel", True),       # one vector as key and value
])
def test_append_matches_pooling(dtype, C, m, W, T, B, gate, shared):
    say("append", dtype, C, m, W, T, B, gate, shared)
    w = I.Workload("t", "csa", seed=71, dtype=dtype, B=B, T=T, m=m, H=8, D=C, W=W, gate=gate)
    raw = {n: v.to(DEV) for n, v in I.draw_raw(w).items()}
    gc = raw["gk"].shape[2]
    wcap = 2 * W
    st = new_state(w, C, gc, wcap, T // m + 1, shared)
    p0 = append_range(st, raw, w, 0, T, 0, shared)
    torch.cuda.synchronize()
    n = T // m
    # the window buffer: positions p0 .. T - 1, bit-exact
    assert max(0, T - wcap) <= p0 <= max(0, T - W)
    for name, src in (("rk", "k"), ("rv", "v" if not shared else "k")):
        assert torch.equal(st[name][:, :T - p0], raw[src][:, p0:T]), name
    for name, src, g in (("ck", "k", "gk"), ("cv", "v", "gv")):
        if shared:
            src, g = "k", "gk"
        got = st[name][:, :n]
        # bit-identical to pooling the whole sequence
        ref_gpu = csa.hca_compress(raw[src].contiguous(), raw[g].contiguous(), m)
        torch.cuda.synchronize()
        assert torch.equal(got, ref_gpu[:, :n]), name
        # and within the bar of the oracle
        ref = oracle.compress(f64(raw[src].cpu()), f64(raw[g].cpu()), m)
        err = maxerr(got, ref)
        say("  ", name, "max err", err)
        assert err <= TOL[dtype]


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_decode_loop_with_append(kind):
    """Per token: append it, then (CSA) index and attend with the caches
    built so far; every step's output against the oracle's attention over the
    whole sequence's caches at that position."""
    m = 4 if kind == "csa" else 16
    H, D, W, k, B = 128, 128, 128, 64, 2
    T0, S = 1500, 24                                # prefix, then S decode steps
    w = I.Workload("t", "csa", seed=72, dtype="bf16", B=B, T=T0 + S, m=m, H=H, D=D, W=W, k=k,
                   Tq=1, q_pos0=T0)
    say("decode loop", kind)
    raw = {n: v.to(DEV) for n, v in I.draw_raw(w).items()}
    C = D
    wcap = 2 * W
    nc_cap = (T0 + S) // m
    st = new_state(w, C, C, wcap, nc_cap, False)
    # the prefix through the same append path (the window then holds its tail)
    p0 = append_range(st, raw, w, 0, T0, 0, False)
    # whole-sequence caches for the oracle
    ck_all = oracle.compress(f64(raw["k"].cpu()), f64(raw["gk"].cpu()), m)
    cv_all = oracle.compress(f64(raw["v"].cpu()), f64(raw["gv"].cpu()), m)
    rk_all, rv_all = f64(raw["k"].cpu()), f64(raw["v"].cpu())
    wq = w.replace(Tq=S, q_pos0=T0)
    q = I.draw_queries(wq, device=DEV)              # [B, S, H, D]
    if kind == "csa":
        kc, ks = csa.csa_quantize_mxfp4(I.draw_indexer_keys(w.replace(T=T0 + S), device=DEV))
        q_idx = I.draw_indexer_queries(wq, device=DEV)
    worst = 0.0
    for s in range(S):
        t = T0 + s
        p0 = append_range(st, raw, w, t, t + 1, p0, False)
        qt = q[:, s:s + 1].contiguous()
        if kind == "csa":
            tk = csa.csa_index_topk(q_idx[:, s:s + 1].contiguous(), kc, ks, m=m, W=W, k=k,
                                    q_pos0=t)
            o = csa.csa_attend(qt, st["ck"], st["cv"], tk, st["rk"], st["rv"], m=m, W=W, q_pos0=t,
                               raw_pos0=p0)
            sel = tk.cpu().numpy()
        else:
            o = csa.hca_attend(qt, st["ck"], st["cv"], st["rk"], st["rv"], m=m, W=W, q_pos0=t,
                               raw_pos0=p0)
            sel = None
        torch.cuda.synchronize()
        ref = oracle.attend(f64(qt.cpu()), ck_all, cv_all, sel, rk_all, rv_all, 0, np.array([t]),
                            m, W)
        err = maxerr(o, ref)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (t, err)
    say("  worst max err", worst)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_decode_loop_mxfp8_entries(kind):
    """The FP8 decode chain per token: append, encode each completed entry to
    MXFP8 (csa_quantize_mxfp8 on its row), attend over the MXFP8 entries and
    the bf16 window; against the oracle's own pooling, encoding and attention
    over the decoded entries."""
    m = 4 if kind == "csa" else 16
    H, D, W, k, B = 128, 128, 128, 64, 2
    T0, S = 1500, 20
    w = I.Workload("t", "csa", seed=73, dtype="bf16", B=B, T=T0 + S, m=m, H=H, D=D, W=W, k=k,
                   Tq=1, q_pos0=T0)
    say("decode loop mxfp8", kind)
    raw = {n: v.to(DEV) for n, v in I.draw_raw(w).items()}
    nc_cap = (T0 + S) // m
    st = new_state(w, D, D, 2 * W, nc_cap, False)
    p0 = append_range(st, raw, w, 0, T0, 0, False)
    kc8, ks8 = csa.csa_quantize_mxfp8(st["ck"])
    vc8, vs8 = csa.csa_quantize_mxfp8(st["cv"])
    ck_all = oracle.compress(f64(raw["k"].cpu()), f64(raw["gk"].cpu()), m)
    cv_all = oracle.compress(f64(raw["v"].cpu()), f64(raw["gv"].cpu()), m)
    ck_dq = oracle.dequant_mxfp8(*oracle.quant_mxfp8(ck_all))
    cv_dq = oracle.dequant_mxfp8(*oracle.quant_mxfp8(cv_all))
    rk_all, rv_all = f64(raw["k"].cpu()), f64(raw["v"].cpu())
    wq = w.replace(Tq=S, q_pos0=T0)
    q = I.draw_queries(wq, device=DEV)
    if kind == "csa":
        kc, ks = csa.csa_quantize_mxfp4(I.draw_indexer_keys(w.replace(T=T0 + S), device=DEV))
        q_idx = I.draw_indexer_queries(wq, device=DEV)
    worst = 0.0
    for s in range(S):
        t = T0 + s
        p0 = append_range(st, raw, w, t, t + 1, p0, False)
        if (t + 1) % m == 0:                          # entry (t + 1) / m - 1 completed
            e = (t + 1) // m - 1
            for b in range(B):
                csa.csa_quantize_mxfp8(st["ck"][b, e:e + 1], codes=kc8[b, e:e + 1],
                                       scales=ks8[b, e:e + 1])
                csa.csa_quantize_mxfp8(st["cv"][b, e:e + 1], codes=vc8[b, e:e + 1],
                                       scales=vs8[b, e:e + 1])
        qt = q[:, s:s + 1].contiguous()
        if kind == "csa":
            tk = csa.csa_index_topk(q_idx[:, s:s + 1].contiguous(), kc, ks, m=m, W=W, k=k,
                                    q_pos0=t)
            o = csa.csa_attend_mxfp8(qt, kc8, vc8, ks8, vs8, tk, st["rk"], st["rv"], m=m, W=W,
                                     q_pos0=t, raw_pos0=p0)
            sel = tk.cpu().numpy()
        else:
            o = csa.hca_attend_mxfp8(qt, kc8, vc8, ks8, vs8, st["rk"], st["rv"], m=m, W=W,
                                     q_pos0=t, raw_pos0=p0)
            sel = None
        torch.cuda.synchronize()
        ref = oracle.attend(f64(qt.cpu()), ck_dq, cv_dq, sel, rk_all, rv_all, 0, np.array([t]),
                            m, W)
        err = maxerr(o, ref)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (t, err)
    say("  worst max err", worst)
