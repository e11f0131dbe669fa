#!/usr/bin/env python3
"""Throughput of the CSA/HCA hot path on one MI355X, with roofline and a
CPU-oracle baseline, printed as one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Workloads (synthetic, seeded, N(0,1); see compressed_sparse_attention_04_amd/inputs.py):
  pair_prefill_128k  (default) one sequence of 131,072 tokens through a CSA
                     layer (m=4, 4-head dim-64 MXFP4 indexer, top-512) and
                     an HCA layer (m'=128), 128 query heads, one shared KV
                     head, head_dim 128, 128-token window, bf16.  A step
                     runs every stage of the path: gated compression of
                     both layers' K and V, MXFP4 encoding of the indexer
                     keys, indexer score + top-k, CSA attention, HCA
                     attention.
  csa_prefill_32k    the CSA layer alone at 32,768 tokens.
  hca_decode_1m      32 sequences x 1,048,576 context tokens, m'=128: the
                     decode step (last-token query over all 8,191
                     candidates + window); caches precompressed, untimed.
  csa_decode_1m      16 sequences x 1,048,576 tokens, m=4: indexer over
                     262,112 candidates + top-512 + attention.

The timed region is exactly K steps bracketed by synchronisations; stage
durations come from HIP events recorded on the launch stream.  Decode
steps rotate over several copies of the caches (> 512 MB in total) so the
256 MB Infinity Cache cannot hold the working set between steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"hbm_GBps": 8000.0, "bf16_TFLOPs": 2500.0, "fp4_TFLOPs": 10100.0}
PIPE_SLICES = 8        # query slices of a pipelined CSA layer (selection | attention)
DEFAULT = "pair_prefill_128k"

# Kernel sources behind each stage: the HBM traffic recorded in
# profiles/traffic.json for a stage is reported only while the digest of
# these sources (comments and blank space removed) still matches.
_IDX = ["indexer.hip", "index_stream.hip", "index_decode.hip", "wave_select.h", "select.h",
        "mxfp4.h", "fp4_tiles.h", "common.h", "internal.h"]
STAGE_SOURCES = {
    "index_topk": _IDX,
    "csa_attend": ["attend.hip", "common.h", "internal.h"],
    "hca_attend": ["attend.hip", "common.h", "internal.h"],
    "compress_m4": ["compress.hip", "common.h", "internal.h"],
    "compress_m128": ["compress.hip", "common.h", "internal.h"],
    "quantize_keys": ["mxfp4.hip", "mxfp4.h", "common.h", "internal.h"],
}


def source_digest(files):
    """sha1 over the kernel sources with comments and blank space removed."""
    import hashlib
    import re
    h = hashlib.sha1()
    for f in files:
        text = open(os.path.join(ROOT, "compressed_sparse_attention_04_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(f.encode())
        h.update(re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()


def recorded_traffic(workload, stage):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE/WRITE_SIZE passes kept
    in profiles/traffic.json, or None if absent or the kernel changed since."""
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
        e = rec["entries"][f"{workload}/{stage}"]
    except (OSError, KeyError, ValueError):
        return None
    if e.get("bytes") is None or e.get("digest") != source_digest(STAGE_SOURCES[stage]):
        return None
    return e["bytes"]


def n_cand(t, m, W):
    """Vectorised candidate count (same rule as the library)."""
    t = np.asarray(t, np.int64)
    w0 = np.maximum(t - W + 1, 0)
    return np.minimum((w0 + m - 1) // m, (t + 1) // m)


def attend_keys(q_pos, m, W, k):
    """Keys each query attends to: kept (k>0) or all (k=0) candidates + window."""
    t = np.asarray(q_pos, np.int64)
    nc = n_cand(t, m, W)
    sel = np.minimum(nc, k) if k > 0 else nc
    nwin = t - np.maximum(t - W + 1, 0) + 1
    return sel + nwin, nc


# --------------------------------------------------------------- workloads
class Stage:
    def __init__(self, name, fn, flops=0.0, bytes_=0.0, peak_key=None, fp4_flops=0.0):
        self.name, self.fn, self.flops, self.bytes, self.peak_key = name, fn, flops, bytes_, peak_key
        self.fp4_flops = fp4_flops        # FP4 indexer flops of a stage that also runs bf16 MFMA


def setup_prefill(dev, layers, shared_kv=False, kv_fmt="bf16", pipeline=False):
    """CSA (and optionally HCA) prefill layers over one sequence.  shared_kv:
    one vector per entry and raw token serves as key and value (only K is
    compressed, and the same buffers are passed as K and V).  kv_fmt
    "mxfp8": the compressed entries are encoded to MXFP8 after pooling (a
    timed stage) and attention reads them in that form.  pipeline (bf16
    entries): a CSA layer's selection and attention run as one
    csa_index_attend call over 8 query slices on two streams."""
    import torch
    from compressed_sparse_attention_04_amd import binding as csa
    from compressed_sparse_attention_04_amd import inputs as I

    stages, tokens, notes = [], None, {}
    for w in layers:
        raw = I.draw_raw(w, device=dev)
        q = I.draw_queries(w, device=dev)
        o = torch.empty_like(q)
        T, D, H, m, W = w.T, w.D, w.H, w.m, w.W
        tokens = w.Tq
        ck = torch.empty((1, w.Nc, D), dtype=q.dtype, device=dev)
        cv = ck if shared_kv else torch.empty_like(ck)
        rv = raw["k"] if shared_kv else raw["v"]
        q_pos = np.arange(w.q_pos0, w.q_pos0 + w.Tq)
        nvec = 1 if shared_kv else 2
        cbytes = nvec * (T * D * 2 + T * D * 2 + w.Nc * D * 2)
        if shared_kv:
            compress = lambda raw=raw, m=m, ck=ck: csa.hca_compress(raw["k"], raw["gk"], m, out=ck)
        else:
            compress = lambda raw=raw, m=m, ck=ck, cv=cv: (
                csa.hca_compress(raw["k"], raw["gk"], m, out=ck),
                csa.hca_compress(raw["v"], raw["gv"], m, out=cv))
        stages.append(Stage(f"compress_m{m}", compress, bytes_=cbytes, peak_key="hbm_GBps"))
        mx = None
        if kv_fmt == "mxfp8":
            kc8 = torch.empty((1, w.Nc, D), dtype=torch.uint8, device=dev)
            ks8 = torch.empty((1, w.Nc, D // 32), dtype=torch.uint8, device=dev)
            vc8, vs8 = (kc8, ks8) if shared_kv else (torch.empty_like(kc8), torch.empty_like(ks8))
            mx = (kc8, vc8, ks8, vs8)

            def encode(ck=ck, cv=cv, mx=mx):
                csa.csa_quantize_mxfp8(ck, codes=mx[0], scales=mx[2])
                if not shared_kv:
                    csa.csa_quantize_mxfp8(cv, codes=mx[1], scales=mx[3])

            stages.append(Stage("encode_mxfp8", encode,
                                bytes_=nvec * w.Nc * (D * 2 + D + D // 32), peak_key="hbm_GBps"))
        if w.kind == "csa":
            k_idx = I.draw_indexer_keys(w, device=dev)
            q_idx = I.draw_indexer_queries(w, device=dev)
            kc = torch.empty((1, w.Nc, w.dI // 2), dtype=torch.uint8, device=dev)
            ks = torch.empty((1, w.Nc, w.dI // 32), dtype=torch.uint8, device=dev)
            topk = torch.empty((1, w.Tq, w.k), dtype=torch.int32, device=dev)
            iws = torch.empty(max(1, csa.csa_index_topk_workspace(1, w.Tq, w.HI, w.dI, w.Nc, m, W,
                                                                  w.k, w.q_pos0)),
                              dtype=torch.uint8, device=dev)
            nkeys, nc = attend_keys(q_pos, m, W, w.k)
            stages.append(Stage("quantize_keys",
                                lambda k_idx=k_idx, kc=kc, ks=ks: csa.csa_quantize_mxfp4(
                                    k_idx, codes=kc, scales=ks),
                                bytes_=w.Nc * (w.dI * 2 + w.dI // 2 + w.dI // 32),
                                peak_key="hbm_GBps"))
            if pipeline and mx is None:
                pws = torch.empty(max(1, csa.csa_index_attend_workspace(
                    1, 1, w.Tq, H, D, w.HI, w.dI, w.Nc, m, W, w.k, w.q_pos0, PIPE_SLICES)),
                    dtype=torch.uint8, device=dev)
                stages.append(Stage(
                    "csa_index_attend",
                    lambda q=q, q_idx=q_idx, kc=kc, ks=ks, ck=ck, cv=cv, raw=raw, rv=rv,
                    topk=topk, o=o, pws=pws, w=w:
                    csa.csa_index_attend(q, q_idx, kc, ks, ck, cv, raw["k"], rv, m=w.m, W=w.W,
                                         k=w.k, q_pos0=w.q_pos0, raw_pos0=0,
                                         n_chunks=PIPE_SLICES, topk=topk, out=o, ws=pws),
                    flops=4.0 * H * D * float(nkeys.sum()), bytes_=2.0 * w.Tq * H * D * 2,
                    peak_key="bf16_TFLOPs", fp4_flops=2.0 * w.HI * w.dI * float(nc.sum())))
                continue
            stages.append(Stage("index_topk",
                                lambda q_idx=q_idx, kc=kc, ks=ks, topk=topk, iws=iws, w=w:
                                csa.csa_index_topk(q_idx, kc, ks, m=w.m, W=w.W, k=w.k,
                                                   q_pos0=w.q_pos0, topk=topk, ws=iws),
                                flops=2.0 * w.HI * w.dI * float(nc.sum()),
                                peak_key="fp4_TFLOPs"))
            if mx is None:
                attend = lambda q=q, ck=ck, cv=cv, topk=topk, raw=raw, rv=rv, o=o, w=w: \
                    csa.csa_attend(q, ck, cv, topk, raw["k"], rv, m=w.m, W=w.W, q_pos0=w.q_pos0,
                                   raw_pos0=0, out=o)
            else:
                attend = lambda q=q, mx=mx, topk=topk, raw=raw, rv=rv, o=o, w=w: \
                    csa.csa_attend_mxfp8(q, mx[0], mx[1], mx[2], mx[3], topk, raw["k"], rv,
                                         m=w.m, W=w.W, q_pos0=w.q_pos0, raw_pos0=0, out=o)
            stages.append(Stage("csa_attend", attend,
                                flops=4.0 * H * D * float(nkeys.sum()),
                                bytes_=2.0 * w.Tq * H * D * 2, peak_key="bf16_TFLOPs"))
        else:
            nkeys, nc = attend_keys(q_pos, m, W, 0)
            if mx is None:
                attend = lambda q=q, ck=ck, cv=cv, raw=raw, rv=rv, o=o, w=w: \
                    csa.hca_attend(q, ck, cv, raw["k"], rv, m=w.m, W=w.W, q_pos0=w.q_pos0,
                                   raw_pos0=0, out=o)
            else:
                attend = lambda q=q, mx=mx, raw=raw, rv=rv, o=o, w=w: \
                    csa.hca_attend_mxfp8(q, mx[0], mx[1], mx[2], mx[3], raw["k"], rv, m=w.m,
                                         W=w.W, q_pos0=w.q_pos0, raw_pos0=0, out=o)
            stages.append(Stage("hca_attend", attend,
                                flops=4.0 * H * D * float(nkeys.sum()),
                                bytes_=2.0 * w.Tq * H * D * 2, peak_key="bf16_TFLOPs"))
    return stages, tokens, notes


def _decode_caches(w, dev, with_keys, shared_kv=False, kv_fmt="bf16"):
    """Precompress every sequence's 1M-token raw context chunk by chunk on the
    GPU; keep the last W raw rows.  Untimed.  shared_kv: K only, passed as
    both K and V."""
    import torch
    from compressed_sparse_attention_04_amd import binding as csa
    from compressed_sparse_attention_04_amd import inputs as I

    L = I.chunk_len(w)
    per = L // w.m
    ck = torch.empty((w.B, w.Nc, w.D), dtype=torch.bfloat16, device=dev)
    cv = ck if shared_kv else torch.empty_like(ck)
    rk = torch.empty((w.B, w.W, w.D), dtype=torch.bfloat16, device=dev)
    rv = rk if shared_kv else torch.empty_like(rk)
    nchunks = w.T // L
    for b in range(w.B):
        for c in range(nchunks):
            x = {n: I.draw_chunk(w, n, b, c, device=dev)[None] for n in ("k", "v", "gk", "gv")}
            csa.hca_compress(x["k"], x["gk"], w.m, out=ck[b:b + 1, c * per:(c + 1) * per])
            if not shared_kv:
                csa.hca_compress(x["v"], x["gv"], w.m, out=cv[b:b + 1, c * per:(c + 1) * per])
            if c == nchunks - 1:
                rk[b].copy_(x["k"][0, -w.W:])
                if not shared_kv:
                    rv[b].copy_(x["v"][0, -w.W:])
    out = {"ck": ck, "cv": cv, "rk": rk, "rv": rv}
    if kv_fmt == "mxfp8":
        out["ck"], out["cks"] = csa.csa_quantize_mxfp8(ck)
        if shared_kv:
            out["cv"], out["cvs"] = out["ck"], out["cks"]
        else:
            out["cv"], out["cvs"] = csa.csa_quantize_mxfp8(cv)
        del ck, cv
    if with_keys:
        k_idx = I.draw_indexer_keys(w, device=dev)
        kc, ks = csa.csa_quantize_mxfp4(k_idx)
        del k_idx
        out["kc"], out["ks"] = kc, ks
    torch.cuda.synchronize()
    return out


def setup_decode(dev, w, min_bytes=600e6, shared_kv=False, kv_fmt="bf16"):
    import torch
    from compressed_sparse_attention_04_amd import binding as csa
    from compressed_sparse_attention_04_amd import inputs as I

    sparse = w.kind == "csa"
    mx8 = kv_fmt == "mxfp8"
    base = _decode_caches(w, dev, sparse, shared_kv, kv_fmt)
    q = I.draw_queries(w, device=dev)
    t = w.q_pos0
    nkeys, nc = attend_keys([t], w.m, w.W, w.k if sparse else 0)
    nwin = min(w.W, t + 1)
    entry_bytes = (w.D + w.D // 32) if mx8 else w.D * 2
    kv_bytes = ((float(nkeys[0]) - nwin) * entry_bytes + nwin * w.D * 2) * (1 if shared_kv else 2)
    qo_bytes = w.H * w.D * 2 * 2
    key_bytes = float(nc[0]) * (w.dI // 2 + w.dI // 32) if sparse else 0.0
    step_bytes = w.B * (kv_bytes + qo_bytes + key_bytes)
    # rotate over enough copies that the step's working set is not cached
    ncopy = max(2, int(np.ceil(min_bytes / step_bytes)) + 1)
    def clone(c):
        d = {n: v.clone() for n, v in c.items()
             if not (shared_kv and n in ("cv", "rv", "cvs"))}
        if shared_kv:
            d["cv"], d["rv"] = d["ck"], d["rk"]
            if mx8:
                d["cvs"] = d["cks"]
        return d

    copies = [base] + [clone(base) for _ in range(ncopy - 1)]
    o = torch.empty_like(q)
    state = {"i": 0}
    stages = []
    if sparse:
        topk = torch.empty((w.B, 1, w.k), dtype=torch.int32, device=dev)
        q_idx = I.draw_indexer_queries(w, device=dev)
        iws = torch.empty(max(1, csa.csa_index_topk_workspace(w.B, 1, w.HI, w.dI, w.Nc, w.m, w.W,
                                                              w.k, t)), dtype=torch.uint8,
                          device=dev)
        aws = torch.empty(max(1, csa.csa_attend_workspace(1, w.B, 1, w.H, w.D, w.k, w.W)),
                          dtype=torch.uint8, device=dev)

        def index():
            c = copies[state["i"] % ncopy]
            csa.csa_index_topk(q_idx, c["kc"], c["ks"], m=w.m, W=w.W, k=w.k, q_pos0=t, topk=topk,
                               ws=iws)

        def attend():
            c = copies[state["i"] % ncopy]
            if mx8:
                csa.csa_attend_mxfp8(q, c["ck"], c["cv"], c["cks"], c["cvs"], topk, c["rk"],
                                     c["rv"], m=w.m, W=w.W, q_pos0=t, raw_pos0=t - w.W + 1,
                                     out=o, ws=aws)
            else:
                csa.csa_attend(q, c["ck"], c["cv"], topk, c["rk"], c["rv"], m=w.m, W=w.W,
                               q_pos0=t, raw_pos0=t - w.W + 1, out=o, ws=aws)
            state["i"] += 1

        stages.append(Stage("index_topk", index, flops=2.0 * w.HI * w.dI * float(nc[0]) * w.B,
                            bytes_=w.B * key_bytes, peak_key="hbm_GBps"))
        stages.append(Stage("csa_attend", attend, flops=4.0 * w.H * w.D * float(nkeys[0]) * w.B,
                            bytes_=w.B * (kv_bytes + qo_bytes), peak_key="hbm_GBps"))
    else:
        aws = torch.empty(max(1, csa.hca_attend_workspace(1, w.B, 1, w.H, w.D, w.Nc, w.m, w.W, t)),
                          dtype=torch.uint8, device=dev)

        def attend():
            c = copies[state["i"] % ncopy]
            if mx8:
                csa.hca_attend_mxfp8(q, c["ck"], c["cv"], c["cks"], c["cvs"], c["rk"], c["rv"],
                                     m=w.m, W=w.W, q_pos0=t, raw_pos0=t - w.W + 1, out=o,
                                     ws=aws)
            else:
                csa.hca_attend(q, c["ck"], c["cv"], c["rk"], c["rv"], m=w.m, W=w.W, q_pos0=t,
                               raw_pos0=t - w.W + 1, out=o, ws=aws)
            state["i"] += 1

        stages.append(Stage("hca_attend", attend, flops=4.0 * w.H * w.D * float(nkeys[0]) * w.B,
                            bytes_=w.B * (kv_bytes + qo_bytes), peak_key="hbm_GBps"))
    return stages, w.B, {"cache_copies": ncopy, "step_bytes": step_bytes}


def setup_stack_decode(dev, n_layers=61, B=16):
    """Decode step of an n-layer attention stack at 1M context: the layer
    schedule of csa_layer_schedule (HCA in layers 0-1, then CSA on even and
    HCA on odd layers), every layer with its own caches (copies of one
    precompressed CSA and one HCA cache set, untimed) and queries, run by one
    csa_stack_attend call."""
    import torch
    from compressed_sparse_attention_04_amd import binding as csa
    from compressed_sparse_attention_04_amd import inputs as I

    wc = I.CSA_DECODE_1M.replace(B=B)
    wh = I.HCA_DECODE_1M.replace(B=B)
    base = {csa.CSA_LAYER_CSA: _decode_caches(wc, dev, True),
            csa.CSA_LAYER_HCA: _decode_caches(wh, dev, False)}
    t = wc.q_pos0
    kinds = csa.csa_layer_schedule(n_layers)
    layers = []
    step_bytes = 0.0
    for l, kind in enumerate(kinds):
        w = (wc if kind == csa.CSA_LAYER_CSA else wh).replace(layer=l)
        c = base[kind] if l == kinds.index(kind) else {n: v.clone() for n, v in base[kind].items()}
        L = {"kind": kind, "m": w.m, "q": I.draw_queries(w, device=dev), "ck": c["ck"],
             "cv": c["cv"], "rk": c["rk"], "rv": c["rv"]}
        L["o"] = torch.empty_like(L["q"])
        nkeys, nc = attend_keys([t], w.m, w.W, w.k if kind == csa.CSA_LAYER_CSA else 0)
        step_bytes += B * (float(nkeys[0]) * w.D * 2 * 2 + w.H * w.D * 2 * 2)
        if kind == csa.CSA_LAYER_CSA:
            L["q_idx"] = I.draw_indexer_queries(w, device=dev)
            L["k_codes"], L["k_scales"] = c["kc"], c["ks"]
            L["topk"] = torch.empty((B, 1, w.k), dtype=torch.int32, device=dev)
            step_bytes += B * float(nc[0]) * (w.dI // 2 + w.dI // 32)
        layers.append(L)
    torch.cuda.synchronize()
    ws = torch.empty(max(1, csa.csa_stack_workspace(1, layers, B, 1, wc.H, wc.D, wc.HI, wc.dI,
                                                    wc.W, wc.k, t)),
                     dtype=torch.uint8, device=dev)

    def run():
        csa.csa_stack_attend(layers, W=wc.W, k=wc.k, q_pos0=t, raw_pos0=t - wc.W + 1,
                             HI=wc.HI, dI=wc.dI, ws=ws)

    stages = [Stage("stack_attend", run, bytes_=step_bytes, peak_key="hbm_GBps")]
    ncsa = kinds.count(csa.CSA_LAYER_CSA)
    return stages, B, {"layers": n_layers, "csa_layers": ncsa, "hca_layers": n_layers - ncsa,
                       "step_bytes": step_bytes}


# --------------------------------------------------------------- CPU baseline
def cpu_baseline(name, budget_s=20.0, n_layers=61):
    """Time the oracle, unchanged, on a bounded sample of the same workload."""
    import torch

    import oracle
    from compressed_sparse_attention_04_amd import inputs as I

    oracle.build()
    cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    f64 = lambda t: t.to(torch.float64).numpy()
    rng = np.random.default_rng(0)

    if name in ("pair_prefill_128k", "csa_prefill_32k"):
        layers = [I.PAIR_CSA_128K, I.PAIR_HCA_128K] if name == "pair_prefill_128k" \
            else [I.CSA_PREFILL_32K]
        per_token = 0.0
        desc = []
        for w in layers:
            nrows = 32
            rows = np.sort(rng.choice(w.Tq, size=nrows, replace=False))
            q_pos = w.q_pos0 + rows
            span = min(w.T, 8192)
            raw = I.draw_raw(w, t0=0, t1=w.T)
            t0 = time.perf_counter()
            oracle.compress(f64(raw["k"][:, :span]), f64(raw["gk"][:, :span]), w.m)
            oracle.compress(f64(raw["v"][:, :span]), f64(raw["gv"][:, :span]), w.m)
            t_comp = (time.perf_counter() - t0) / span
            # the sampled rows need the full compressed cache (not timed)
            ck = oracle.compress(f64(raw["k"]), f64(raw["gk"]), w.m)
            cv = oracle.compress(f64(raw["v"]), f64(raw["gv"]), w.m)
            q = f64(I.draw_queries(w, rows=rows))
            t0 = time.perf_counter()
            if w.kind == "csa":
                kc, ks = oracle.quant_mxfp4(f64(I.draw_indexer_keys(w)))
                tk, _ = oracle.index_topk(f64(I.draw_indexer_queries(w, rows=rows)), kc, ks, q_pos,
                                          w.m, w.W, w.k)
            else:
                tk = None
            oracle.attend(q, ck, cv, tk, f64(raw["k"]), f64(raw["v"]), 0, q_pos, w.m, w.W)
            t_rows = (time.perf_counter() - t0) / nrows
            per_token += t_comp + t_rows
            desc.append(f"{w.name}: compression of {span} tokens + index/attend of {nrows} "
                        f"random query rows")
        return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                "sample": "; ".join(desc) + " (per-token times summed over the layers)"}

    def decode_seconds(w):
        """The oracle's decode step of one sequence of workload w."""
        ws = w.replace(B=1)
        t = w.q_pos0
        ck = f64(I.draw_cache(ws, "ck", w.Nc))
        cv = f64(I.draw_cache(ws, "cv", w.Nc))
        rk = f64(I.draw_cache(ws, "rk", w.W))
        rv = f64(I.draw_cache(ws, "rv", w.W))
        q = f64(I.draw_queries(ws))
        t0 = time.perf_counter()
        if w.kind == "csa":
            kc, ks = oracle.quant_mxfp4(f64(I.draw_indexer_keys(ws)))
            t0 = time.perf_counter()
            tk, _ = oracle.index_topk(f64(I.draw_indexer_queries(ws)), kc, ks, [t], w.m, w.W, w.k)
        else:
            tk = None
        oracle.attend(q, ck, cv, tk, rk, rv, t - w.W + 1, [t], w.m, w.W)
        return time.perf_counter() - t0

    if name == "stack_decode_1m":
        from compressed_sparse_attention_04_amd import binding as csa
        kinds = csa.csa_layer_schedule(n_layers)
        ncsa = kinds.count(csa.CSA_LAYER_CSA)
        t_csa = decode_seconds(I.CSA_DECODE_1M)
        t_hca = decode_seconds(I.HCA_DECODE_1M)
        return {"value": 1.0 / (ncsa * t_csa + (n_layers - ncsa) * t_hca), "unit": "tokens/s",
                "cores": threads, "kind": "oracle",
                "sample": f"one sequence's decode step of one CSA and one HCA layer, scaled to "
                          f"{ncsa} CSA + {n_layers - ncsa} HCA layers"}
    w = I.HCA_DECODE_1M if name == "hca_decode_1m" else I.CSA_DECODE_1M
    el = decode_seconds(w)
    return {"value": 1.0 / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "decode step of 1 sequence (caches drawn at the workload's shapes)"}


# --------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default=DEFAULT,
                    choices=["pair_prefill_128k", "csa_prefill_32k", "hca_decode_1m",
                             "csa_decode_1m", "stack_decode_1m"])
    ap.add_argument("--layers", type=int, default=61,
                    help="layers of the stack_decode_1m workload (default 61)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shared-kv", action="store_true",
                    help="one vector per compressed entry and raw token serves as key and "
                         "value (the same buffers passed as K and V); default: separate K, V")
    ap.add_argument("--kv-format", default="bf16", choices=["bf16", "mxfp8"],
                    help="storage of the compressed entries: bf16 (default) or MXFP8 E4M3 "
                         "codes with a power-of-two scale per 32 values (the raw window "
                         "stays bf16)")
    ap.add_argument("--pipeline", action="store_true",
                    help="run a CSA prefill layer's selection and attention as one "
                         "csa_index_attend call, pipelined over query slices on two streams "
                         "(default: two stages in order)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy three times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the path has no multi-GPU mode (sequences or "
              "query ranges would shard across GPUs); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = "cuda:0"
    torch.cuda.set_device(0)
    from compressed_sparse_attention_04_amd import inputs as I

    decode = args.workload.endswith("decode_1m")
    steps = args.steps if args.steps is not None else (50 if decode else 10)
    warmup = args.warmup if args.warmup is not None else (5 if decode else 2)

    if args.workload == "pair_prefill_128k":
        stages, tokens, notes = setup_prefill(dev, [I.PAIR_CSA_128K, I.PAIR_HCA_128K],
                                              args.shared_kv, args.kv_format,
                                              args.pipeline)
        wl = {"workload": "csa_hca_layer_pair_prefill", "seq_len": 131072, "batch": 1,
              "heads": 128, "kv_heads": 1, "head_dim": 128, "m_csa": 4, "m_hca": 128,
              "top_k": 512, "indexer": "4x64 MXFP4", "window": 128}
        metric, unit = "prefill tokens/s", "tokens/s"
    elif args.workload == "csa_prefill_32k":
        stages, tokens, notes = setup_prefill(dev, [I.CSA_PREFILL_32K], args.shared_kv,
                                              args.kv_format, args.pipeline)
        wl = {"workload": "csa_prefill", "seq_len": 32768, "batch": 1, "heads": 128,
              "kv_heads": 1, "head_dim": 128, "m": 4, "top_k": 512, "indexer": "4x64 MXFP4",
              "window": 128}
        metric, unit = "prefill tokens/s", "tokens/s"
    elif args.workload == "stack_decode_1m":
        if args.kv_format != "bf16" or args.shared_kv:
            print("stack_decode_1m runs bf16 caches with separate K and V", file=sys.stderr)
            sys.exit(2)
        stages, tokens, notes = setup_stack_decode(dev, args.layers)
        wc = I.CSA_DECODE_1M
        wl = {"workload": "attention_stack_decode_1m_ctx", "context": wc.T, "batch": tokens,
              "layers": notes["layers"], "csa_layers": notes["csa_layers"],
              "hca_layers": notes["hca_layers"], "heads": wc.H, "kv_heads": 1,
              "head_dim": wc.D, "m_csa": 4, "m_hca": 128, "top_k": wc.k, "window": wc.W}
        metric, unit = "1M-ctx decode tokens/s/GPU (attention stack)", "tokens/s"
    else:
        w = I.HCA_DECODE_1M if args.workload == "hca_decode_1m" else I.CSA_DECODE_1M
        stages, tokens, notes = setup_decode(dev, w, shared_kv=args.shared_kv,
                                             kv_fmt=args.kv_format)
        wl = {"workload": args.workload.replace("_1m", "") + "_1m_ctx", "context": w.T,
              "batch": w.B, "heads": w.H, "kv_heads": 1, "head_dim": w.D, "m": w.m,
              "top_k": w.k if w.kind == "csa" else None, "window": w.W}
        metric, unit = "1M-ctx decode tokens/s/GPU", "tokens/s"
    if not decode and args.pipeline and args.kv_format == "bf16":
        wl["csa_schedule"] = (f"selection and attention pipelined over {PIPE_SLICES} query "
                              "slices on two streams (csa_index_attend)")
    wl["kv"] = "one vector as key and value" if args.shared_kv else "separate K and V"
    wl["kv_format"] = ("compressed entries MXFP8 (E4M3), window bf16" if args.kv_format == "mxfp8"
                       else "bf16")

    stream = torch.cuda.current_stream()

    def step(ev=None):
        for si, st in enumerate(stages):
            st.fn()
            if ev is not None:
                ev[si].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in stages] for _ in range(steps)]
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        starts[s].record(stream)
        step(evs[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    stage_ms = np.zeros(len(stages))
    for s in range(steps):
        prev = starts[s]
        for si in range(len(stages)):
            stage_ms[si] += prev.elapsed_time(evs[s][si])
            prev = evs[s][si]
    stage_ms /= steps
    ms_per_step = elapsed * 1e3 / steps
    value = tokens / (ms_per_step / 1e3)

    dom = int(np.argmax(stage_ms))
    d = stages[dom]
    sec = stage_ms[dom] / 1e3
    if d.peak_key == "hbm_GBps":
        roof = {"bound": "hbm", "achieved": d.bytes / sec / 1e9, "peak": PEAK["hbm_GBps"],
                "unit": "GB/s"}
    else:
        # a pipelined CSA layer runs FP4 indexer and bf16 attention MFMAs side by
        # side: its FP4 flops count at the bf16/FP4 peak ratio, so achieved/peak
        # is the sum over both of (flops / own peak) / time
        eq = d.flops + d.fp4_flops * PEAK["bf16_TFLOPs"] / PEAK["fp4_TFLOPs"]
        roof = {"bound": "mfma", "achieved": eq / sec / 1e12, "peak": PEAK[d.peak_key],
                "unit": "TFLOP/s"}
        if d.fp4_flops:
            roof["convention"] = ("bf16-equivalent: attention bf16 flops + indexer FP4 flops x "
                                  "2.5/10.1")
    roof["frac"] = roof["achieved"] / roof["peak"]
    # (counter passes exist for the default inputs only)
    roof["traffic"] = (None if args.shared_kv or args.kv_format != "bf16"
                       else recorded_traffic(args.workload, d.name))
    roof["kernel"] = d.name
    roof["ms_per_launch"] = stage_ms[dom]

    stage_info = {}
    for st, ms in zip(stages, stage_ms):
        e = {"ms": round(float(ms), 4)}
        if st.flops:
            e["TFLOP/s"] = round(st.flops / (ms / 1e3) / 1e12, 2)
        if st.fp4_flops:
            e["indexer FP4 TFLOP/s"] = round(st.fp4_flops / (ms / 1e3) / 1e12, 2)
        if st.bytes:
            e["GB/s"] = round(st.bytes / (ms / 1e3) / 1e9, 1)
        stage_info[st.name] = e

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, n_layers=args.layers)

    rec = {"metric": metric, "value": round(value, 1), "unit": unit, "n_gpus": 1,
           "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1))", "config": wl, "roofline": roof,
           "cpu_baseline": cpu, "stages": stage_info}
    rec.update({k: v for k, v in notes.items()})
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
