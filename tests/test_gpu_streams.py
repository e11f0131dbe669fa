"""Calls on a stream other than the current one: every entry point of a CSA
and an HCA layer (pooling, key encoding, selection, attention) launched on a
side stream gives results bit-identical to the same calls on the current
stream.  The tensors and workspaces the binding allocates for such a call are
marked as used by the side stream, so allocations made on the current stream
while the side stream still runs must not take their memory; the test makes
such allocations, and writes them, before it waits for the side stream."""
import pytest
import torch

from compressed_sparse_attention_04_amd import binding as csa
from compressed_sparse_attention_04_amd import inputs as I
from tests.gpu_helpers import DEV, say

pytestmark = pytest.mark.gpu


def _layer(w, raw, k_idx, qi, q, stream):
    """Pooling, key encoding, selection and attention of a CSA layer (m = 4)
    and attention of an HCA layer (m' = 128) over the same raw rows, all with
    the binding's own allocations, on `stream` (None: the current stream)."""
    ck = csa.hca_compress(raw["k"], raw["gk"], 4, stream=stream)
    cv = csa.hca_compress(raw["v"], raw["gv"], 4, stream=stream)
    kc, ks = csa.csa_quantize_mxfp4(k_idx, stream=stream)
    tk = csa.csa_index_topk(qi, kc, ks, m=4, W=w.W, k=w.k, q_pos0=w.q_pos0, stream=stream)
    o = csa.csa_attend(q, ck, cv, tk, raw["k"], raw["v"], m=4, W=w.W, q_pos0=w.q_pos0,
                       raw_pos0=0, stream=stream)
    hk = csa.hca_compress(raw["k"], raw["gk"], 128, stream=stream)
    hv = csa.hca_compress(raw["v"], raw["gv"], 128, stream=stream)
    oh = csa.hca_attend(q, hk, hv, raw["k"], raw["v"], m=128, W=w.W, q_pos0=w.q_pos0,
                        raw_pos0=0, stream=stream)
    return [ck, cv, kc, ks, tk, o, hk, hv, oh]


@pytest.mark.parametrize("T,q0,Tq,B", [
    (6000, 5000, 64, 1),        # prefill rows: streaming selection, one attention split
    (4 * 70000, 4 * 70000 - 1, 1, 2),   # decode rows: chunked selection, split attention
])
def test_side_stream_matches_current_stream(T, q0, Tq, B):
    say("side stream", T, q0, Tq, B)
    w = I.Workload("t", "csa", seed=91, dtype="bf16", B=B, T=T, m=4, H=128, D=128, W=128,
                   k=512, Tq=Tq, q_pos0=q0)
    raw = {n: t.to(DEV) for n, t in I.draw_raw(w).items()}
    k_idx = I.draw_indexer_keys(w, device=DEV)
    qi = I.draw_indexer_queries(w, device=DEV)
    q = I.draw_queries(w, device=DEV)
    ref = _layer(w, raw, k_idx, qi, q, None)
    torch.cuda.synchronize()

    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    got = _layer(w, raw, k_idx, qi, q, side)
    # work on the current stream while the side stream may still run: fresh
    # allocations there must not reuse what the side stream's calls hold
    junk = [torch.full((1 << 20,), -7, dtype=torch.int32, device=DEV) for _ in range(16)]
    for j in junk:
        j.add_(1)
    side.synchronize()
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    assert all(bool((j == -6).all()) for j in junk)
