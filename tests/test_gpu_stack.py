"""A stack of CSA/HCA layers through csa_stack_attend on the GPU.

Each layer has its own caches, indexer keys and queries (seeded by layer).
Checked per layer: the stack's outputs and selections are bit-identical to
the same layer run through the single-layer entry points, the CSA
selections equal the oracle's top-k, and the outputs are within the bf16
bar of the oracle's attention."""
import numpy as np
import pytest
import torch

import oracle
from compressed_sparse_attention_04_amd import binding as csa
from compressed_sparse_attention_04_amd import inputs as I
from tests.gpu_helpers import DEV, TOL, f64, maxerr, say

pytestmark = pytest.mark.gpu


def build_layers(n_layers, B, T, Tq, q_pos0, W, k, raw_pos0, raw_len, seed=61):
    kinds = csa.csa_layer_schedule(n_layers)
    layers, host = [], []
    for l, kind in enumerate(kinds):
        csa_layer = kind == csa.CSA_LAYER_CSA
        m = 4 if csa_layer else 128
        w = I.Workload("t", "csa" if csa_layer else "hca", seed=seed, dtype="bf16", B=B, T=T, m=m,
                       H=128, D=128, W=W, k=k if csa_layer else 0, Tq=Tq, q_pos0=q_pos0, layer=l)
        Nc = T // m
        h = {"kind": kind, "m": m, "q": I.draw_queries(w), "ck": I.draw_cache(w, "ck", Nc),
             "cv": I.draw_cache(w, "cv", Nc)}
        rk, rv = I.draw_cache(w, "rk", raw_pos0 + raw_len), I.draw_cache(w, "rv", raw_pos0 + raw_len)
        h["rk"], h["rv"] = rk[:, raw_pos0:].contiguous(), rv[:, raw_pos0:].contiguous()
        if csa_layer:
            h["q_idx"] = I.draw_indexer_queries(w)
            h["k_codes"], h["k_scales"] = oracle.quant_mxfp4(f64(I.draw_indexer_keys(w)))
        d = {n: (torch.from_numpy(v) if isinstance(v, np.ndarray) else v).to(DEV)
             for n, v in h.items() if n not in ("kind", "m")}
        d.update(kind=kind, m=m, o=torch.empty_like(d["q"]))
        if csa_layer:
            d["topk"] = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
        layers.append(d)
        host.append(h)
    return layers, host


@pytest.mark.parametrize("n_layers,B,T,Tq,q_pos0,W,k,decode", [
    (5, 2, 3000, 9, 2900, 128, 64, False),        # prefill rows, ragged tiles
    (6, 3, 20000, 1, 19999, 128, 512, True),      # decode: window-only raw rows, splits
])
def test_stack_matches_layers_and_oracle(n_layers, B, T, Tq, q_pos0, W, k, decode):
    say("stack", n_layers, B, T, Tq, q_pos0, W, k, decode)
    raw_pos0 = q_pos0 - W + 1 if decode else 0
    raw_len = W if decode else T
    layers, host = build_layers(n_layers, B, T, Tq, q_pos0, W, k, raw_pos0, raw_len)
    csa.csa_stack_attend(layers, W=W, k=k, q_pos0=q_pos0, raw_pos0=raw_pos0)
    torch.cuda.synchronize()
    q_pos = np.arange(q_pos0, q_pos0 + Tq)
    for l, (d, h) in enumerate(zip(layers, host)):
        m = d["m"]
        if d["kind"] == csa.CSA_LAYER_CSA:
            tk = csa.csa_index_topk(d["q_idx"], d["k_codes"], d["k_scales"], m=m, W=W, k=k,
                                    q_pos0=q_pos0)
            one = csa.csa_attend(d["q"], d["ck"], d["cv"], tk, d["rk"], d["rv"], m=m, W=W,
                                 q_pos0=q_pos0, raw_pos0=raw_pos0)
            torch.cuda.synchronize()
            assert torch.equal(d["topk"], tk), l
            ref_tk, _ = oracle.index_topk(f64(h["q_idx"]), h["k_codes"], h["k_scales"], q_pos, m,
                                          W, k)
            assert np.array_equal(d["topk"].cpu().numpy(), ref_tk), l
            sel = ref_tk
        else:
            one = csa.hca_attend(d["q"], d["ck"], d["cv"], d["rk"], d["rv"], m=m, W=W,
                                 q_pos0=q_pos0, raw_pos0=raw_pos0)
            torch.cuda.synchronize()
            sel = None
        assert torch.equal(d["o"], one), l
        ref = oracle.attend(f64(h["q"]), f64(h["ck"]), f64(h["cv"]), sel, f64(h["rk"]),
                            f64(h["rv"]), raw_pos0, q_pos, m, W)
        err = maxerr(d["o"], ref)
        say("  layer", l, "kind", d["kind"], "max err", err)
        assert err <= TOL["bf16"]
