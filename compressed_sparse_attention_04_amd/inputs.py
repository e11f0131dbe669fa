"""Seeded synthetic inputs and the workload shapes they are drawn for.

This module holds no arithmetic of the method: it only draws N(0,1) numbers
with fixed seeds, scales them and rounds them to the storage dtype.  It is
the one piece shared by the GPU path's tests and benchmark and by the CPU
oracle's callers.

Every tensor is drawn from its own generator whose seed is a function of
(workload seed, layer, tensor name, sequence, chunk).  Long contexts are
therefore drawn chunk by chunk and any chunk can be drawn again on its own.
Draws are made in float32 and then rounded (round-to-nearest-even) to the
workload dtype.  The same seed gives the same numbers on the same device
type; CPU and GPU generators give different streams.
"""
from __future__ import annotations

import dataclasses
import math

import torch

# Tensor names: raw K/V rows, their gate logits, the indexer key/query
# inputs, the attention query, and directly-drawn compressed or raw caches
# used by stage-wise tests.
_TENSOR_IDS = {"k": 1, "v": 2, "gk": 3, "gv": 4, "k_idx": 5, "q_idx": 6, "q": 7,
               "ck": 8, "cv": 9, "rk": 10, "rv": 11, "g": 12, "topk_perm": 13}

CHUNK = 65536          # tokens per drawn chunk of a long context


def subseed(seed: int, name: str, layer: int = 0, seq: int = 0, chunk: int = 0) -> int:
    s = seed
    for v in (layer, _TENSOR_IDS[name], seq, chunk):
        s = (s * 1_000_003 + v + 1) % (1 << 61)
    return s


def normal(shape, seed: int, name: str, *, layer: int = 0, seq: int = 0, chunk: int = 0,
           scale: float = 1.0, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """N(0,1) * scale drawn in float32 from a dedicated generator, then rounded
    to ``dtype``."""
    g = torch.Generator(device=device)
    g.manual_seed(subseed(seed, name, layer, seq, chunk))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention layer's problem shape.

    kind        "csa" (indexer + top-k + sparse attention) or "hca" (dense)
    B, T        sequences and context length (tokens per sequence)
    m           compression ratio (block length)
    H, D        query heads and head dim (one shared K/V head)
    W           sliding-window length
    HI, dI, k   indexer heads, indexer dim, kept entries (csa only)
    Tq, q_pos0  query rows per sequence and the position of the first
    gate        "token" ([T,1], shared by K and V) or "channel" ([T,D] each)
    """
    name: str
    kind: str
    seed: int
    dtype: str
    B: int
    T: int
    m: int
    H: int
    D: int
    W: int = 128
    HI: int = 4
    dI: int = 64
    k: int = 512
    Tq: int = 0
    q_pos0: int = 0
    gate: str = "channel"
    layer: int = 0

    @property
    def Nc(self) -> int:
        return self.T // self.m

    @property
    def q_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five problem shapes of the workloads (seeded, N(0,1) data):
TINY_CSA = Workload("tiny_csa_f32", "csa", seed=0, dtype="f32", B=1, T=1024, m=4, H=8, D=64,
                    W=128, HI=2, dI=32, k=16, Tq=16, q_pos0=1008, gate="token")
CSA_PREFILL_32K = Workload("csa_prefill_32k_bf16", "csa", seed=1, dtype="bf16", B=1, T=32768,
                           m=4, H=128, D=128, Tq=32768, q_pos0=0)
HCA_DECODE_1M = Workload("hca_decode_1m_b32_bf16", "hca", seed=2, dtype="bf16", B=32,
                         T=1 << 20, m=128, H=128, D=128, k=0, Tq=1, q_pos0=(1 << 20) - 1)
CSA_DECODE_1M = Workload("csa_decode_1m_b16_bf16", "csa", seed=3, dtype="bf16", B=16,
                         T=1 << 20, m=4, H=128, D=128, Tq=1, q_pos0=(1 << 20) - 1)
PAIR_CSA_128K = Workload("pair_prefill_128k_csa", "csa", seed=4, dtype="bf16", B=1, T=131072,
                         m=4, H=128, D=128, Tq=131072, q_pos0=0, layer=0)
PAIR_HCA_128K = Workload("pair_prefill_128k_hca", "hca", seed=4, dtype="bf16", B=1, T=131072,
                         m=128, H=128, D=128, k=0, Tq=131072, q_pos0=0, layer=1)

WORKLOADS = {w.name: w for w in (TINY_CSA, CSA_PREFILL_32K, HCA_DECODE_1M, CSA_DECODE_1M,
                                 PAIR_CSA_128K, PAIR_HCA_128K)}


def chunk_len(w: Workload) -> int:
    """Tokens per drawn chunk of a raw tensor of this workload."""
    return min(CHUNK, w.T)


def _raw_name(w: Workload, name: str) -> str:
    # a per-token gate is one logit per token shared by K and V
    if w.gate == "token" and name in ("gk", "gv"):
        return "g"
    return name


def _raw_cols(w: Workload, name: str) -> int:
    return 1 if _raw_name(w, name) == "g" else w.D


def draw_chunk(w: Workload, name: str, seq: int, chunk: int, device="cpu") -> torch.Tensor:
    """Chunk ``chunk`` of raw tensor ``name`` ("k", "v", "gk", "gv") of
    sequence ``seq``: [chunk_len(w), D] (or [chunk_len(w), 1] for a per-token
    gate).  A sequence's rows are the concatenation of its chunks."""
    return normal((chunk_len(w), _raw_cols(w, name)), w.seed, _raw_name(w, name),
                  layer=w.layer, seq=seq, chunk=chunk, dtype=torch_dtype(w.dtype),
                  device=device)


def draw_rows(w: Workload, name: str, seq: int, t0: int, t1: int, device="cpu") -> torch.Tensor:
    """Rows [t0, t1) of raw tensor ``name`` of sequence ``seq``."""
    L = chunk_len(w)
    parts = []
    for c in range(t0 // L, (t1 - 1) // L + 1):
        x = draw_chunk(w, name, seq, c, device)
        lo = max(t0 - c * L, 0)
        hi = min(t1 - c * L, L)
        parts.append(x[lo:hi])
    return torch.cat(parts) if len(parts) > 1 else parts[0]


def draw_raw(w: Workload, device="cpu", t0: int = 0, t1: int | None = None):
    """Raw K, V and gate rows of positions [t0, t1) for every sequence:
    {"k","v","gk","gv"} -> [B, t1-t0, D or 1]."""
    t1 = w.T if t1 is None else t1
    return {name: torch.stack([draw_rows(w, name, b, t0, t1, device) for b in range(w.B)])
            for name in ("k", "v", "gk", "gv")}


def draw_indexer_keys(w: Workload, device="cpu", rows: int | None = None) -> torch.Tensor:
    """Indexer key inputs, one dI-vector per compressed entry: [B, Nc, dI]."""
    n = w.Nc if rows is None else rows
    return torch.stack([normal((n, w.dI), w.seed, "k_idx", layer=w.layer, seq=b,
                               dtype=torch_dtype(w.dtype), device=device) for b in range(w.B)])


QCHUNK = 1024         # query rows per drawn chunk of the query tensors


def _draw_query_rows(w: Workload, name: str, row_shape, scale: float, device, rows):
    """Rows of a per-query tensor drawn in chunks of QCHUNK query rows, so a
    few sampled rows can be drawn without drawing all of them."""
    dt = torch_dtype(w.dtype)
    if rows is None:
        rows = torch.arange(w.Tq)
    rows = torch.as_tensor(rows, dtype=torch.int64).cpu()
    out = []
    for b in range(w.B):
        parts = {}
        for c in sorted(set((rows // QCHUNK).tolist())):
            n = min(QCHUNK, w.Tq - c * QCHUNK)
            parts[c] = normal((n,) + tuple(row_shape), w.seed, name, layer=w.layer, seq=b,
                              chunk=c, scale=scale, dtype=dt, device=device)
        if len(rows) == w.Tq and torch.equal(rows, torch.arange(w.Tq)):
            out.append(torch.cat([parts[c] for c in sorted(parts)]))
        else:
            out.append(torch.stack([parts[int(r) // QCHUNK][int(r) % QCHUNK] for r in rows]))
    return torch.stack(out)


def draw_indexer_queries(w: Workload, device="cpu", rows=None) -> torch.Tensor:
    """Indexer query inputs [B, Tq, HI, dI] (or only the query rows ``rows``)."""
    return _draw_query_rows(w, "q_idx", (w.HI, w.dI), 1.0, device, rows)


def draw_queries(w: Workload, device="cpu", rows=None) -> torch.Tensor:
    """Attention queries [B, Tq, H, D], N(0,1) * 1/sqrt(D) rounded to dtype
    (or only the query rows ``rows``)."""
    return _draw_query_rows(w, "q", (w.H, w.D), w.q_scale, device, rows)


def draw_cache(w: Workload, name: str, rows: int, device="cpu") -> torch.Tensor:
    """A directly drawn [B, rows, D] cache (``ck``, ``cv``, ``rk`` or ``rv``)
    for stage-wise tests of the attention step."""
    return torch.stack([normal((rows, w.D), w.seed, name, layer=w.layer, seq=b,
                               dtype=torch_dtype(w.dtype), device=device) for b in range(w.B)])
