"""csa_index_topk_noalloc (static scratch, no workspace argument) against
csa_index_topk with a workspace: identical indices on two calls in a row,
the second over a smaller input, through the C ABI."""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_04_amd import binding as csa
from compressed_sparse_attention_04_amd import inputs as I
from gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


def case(B, T, Tq, k, seed):
    w = I.Workload("t", "csa", seed=seed, dtype="bf16", B=B, T=T, m=4, H=128, D=128, k=k)
    w = w.replace(Tq=Tq, q_pos0=T - Tq)
    kc, ks = csa.csa_quantize_mxfp4(I.draw_indexer_keys(w).to(DEV))
    q_idx = I.draw_indexer_queries(w).to(DEV)
    return w, q_idx, kc, ks


def test_noalloc_matches_workspace_call_twice():
    # decode rows over 262,112 candidates (the scratch holds their chunk
    # lists), then a smaller decode problem that reuses the same scratch
    for (B, T, Tq, k, seed) in [(16, 4 * 262144, 1, 512, 41), (3, 4 * 50000, 2, 256, 42)]:
        say("noalloc", B, T, Tq, k)
        w, q_idx, kc, ks = case(B, T, Tq, k, seed)
        ref = csa.csa_index_topk(q_idx, kc, ks, m=w.m, W=w.W, k=w.k, q_pos0=w.q_pos0)
        out = torch.full_like(ref, -7)
        got = csa.csa_index_topk_noalloc(q_idx, kc, ks, m=w.m, W=w.W, k=w.k, q_pos0=w.q_pos0,
                                         topk=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())


def test_noalloc_prefill_rows_without_scratch():
    # rows over <= 32,768 candidates need no scratch at all
    say("noalloc prefill rows")
    w, q_idx, kc, ks = case(1, 40000, 20, 512, 43)
    ref = csa.csa_index_topk(q_idx, kc, ks, m=w.m, W=w.W, k=w.k, q_pos0=w.q_pos0)
    got = csa.csa_index_topk_noalloc(q_idx, kc, ks, m=w.m, W=w.W, k=w.k, q_pos0=w.q_pos0)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())


def test_noalloc_refuses_oversized_selection():
    say("noalloc oversize")
    w, q_idx, kc, ks = case(1, 140000, 300, 512, 44)       # chunk lists > 4 MiB
    with pytest.raises(csa.CsaError, match="scratch"):
        csa.csa_index_topk_noalloc(q_idx, kc, ks, m=w.m, W=w.W, k=w.k, q_pos0=w.q_pos0)
