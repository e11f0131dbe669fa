"""The decode step captured in a HIP graph (as a serving loop would capture
it) gives exactly the eager results on every replay, with the program's own
eager work and synchronisations between replays: the entry points allocate
nothing, synchronise nothing and record no memset node."""
import pytest
import torch

from compressed_sparse_attention_04_amd import binding as csa
from compressed_sparse_attention_04_amd import inputs as I
from tests.gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


def _decode_inputs(kind, seed):
    mx8 = kind.endswith("_mxfp8")
    kind = kind.split("_")[0]
    m = 4 if kind == "csa" else 128
    T = m * 3000
    w = I.Workload("graph", kind, seed=seed, dtype="bf16", B=2, T=T, m=m, H=128, D=128, W=128,
                   k=512, Tq=1, q_pos0=T - 1)
    t = w.q_pos0
    d = {"q": I.draw_queries(w, device=DEV),
         "ck": I.draw_cache(w, "ck", w.Nc, device=DEV),
         "cv": I.draw_cache(w, "cv", w.Nc, device=DEV),
         "rk": I.draw_cache(w, "rk", w.W, device=DEV),
         "rv": I.draw_cache(w, "rv", w.W, device=DEV)}
    if kind == "csa":
        d["kc"], d["ks"] = csa.csa_quantize_mxfp4(I.draw_indexer_keys(w, device=DEV))
        d["q_idx"] = I.draw_indexer_queries(w, device=DEV)
        d["topk"] = torch.empty((w.B, 1, w.k), dtype=torch.int32, device=DEV)
        d["iws"] = torch.empty(max(1, csa.csa_index_topk_workspace(w.B, 1, w.HI, w.dI, w.Nc, w.m,
                                                                   w.W, w.k, t)),
                               dtype=torch.uint8, device=DEV)
        d["aws"] = torch.empty(max(1, csa.csa_attend_workspace(1, w.B, 1, w.H, w.D, w.k, w.W)),
                               dtype=torch.uint8, device=DEV)
    else:
        d["aws"] = torch.empty(max(1, csa.hca_attend_workspace(1, w.B, 1, w.H, w.D, w.Nc, w.m,
                                                               w.W, t)),
                               dtype=torch.uint8, device=DEV)
    d["o"] = torch.empty_like(d["q"])
    if mx8:                                       # MXFP8 compressed entries (encoded eagerly)
        d["ck"], d["cks"] = csa.csa_quantize_mxfp8(d["ck"])
        d["cv"], d["cvs"] = csa.csa_quantize_mxfp8(d["cv"])
    return w, d


def _step(kind, w, d):
    t = w.q_pos0
    mx8 = kind.endswith("_mxfp8")
    if kind.startswith("csa"):
        csa.csa_index_topk(d["q_idx"], d["kc"], d["ks"], m=w.m, W=w.W, k=w.k, q_pos0=t,
                           topk=d["topk"], ws=d["iws"])
        if mx8:
            csa.csa_attend_mxfp8(d["q"], d["ck"], d["cv"], d["cks"], d["cvs"], d["topk"],
                                 d["rk"], d["rv"], m=w.m, W=w.W, q_pos0=t, raw_pos0=t - w.W + 1,
                                 out=d["o"], ws=d["aws"])
        else:
            csa.csa_attend(d["q"], d["ck"], d["cv"], d["topk"], d["rk"], d["rv"], m=w.m, W=w.W,
                           q_pos0=t, raw_pos0=t - w.W + 1, out=d["o"], ws=d["aws"])
    elif mx8:
        csa.hca_attend_mxfp8(d["q"], d["ck"], d["cv"], d["cks"], d["cvs"], d["rk"], d["rv"],
                             m=w.m, W=w.W, q_pos0=t, raw_pos0=t - w.W + 1, out=d["o"],
                             ws=d["aws"])
    else:
        csa.hca_attend(d["q"], d["ck"], d["cv"], d["rk"], d["rv"], m=w.m, W=w.W, q_pos0=t,
                       raw_pos0=t - w.W + 1, out=d["o"], ws=d["aws"])


@pytest.mark.parametrize("kind", ["csa", "hca", "csa_mxfp8", "hca_mxfp8"])
def test_decode_step_graph_replay(kind):
    say("graph replay", kind)
    w, d = _decode_inputs(kind, seed=71)
    _step(kind, w, d)
    torch.cuda.synchronize()
    ref_o = d["o"].clone()
    ref_tk = d["topk"].clone() if kind.startswith("csa") else None
    # other eager work between the replays: the same step on other inputs
    w2, d2 = _decode_inputs(kind, seed=72)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(kind, w, d)
    for r in range(3):
        d["o"].fill_(0)
        if kind.startswith("csa"):
            d["topk"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["o"], ref_o), f"replay {r}: attention output differs"
        if kind.startswith("csa"):
            assert torch.equal(d["topk"], ref_tk), f"replay {r}: kept set differs"
        _step(kind, w2, d2)
        torch.cuda.synchronize()
