"""ctypes binding of libcsa.so (include/csa.h): the same entry points, taking
torch device tensors.  Argument marshalling only -- every step runs in the
library's HIP kernels; torch provides device memory and the stream.

Importing this module does not load the library; the first call does, and
raises :class:`CsaError` if ``libcsa.so`` has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa.so")

CSA_F32, CSA_BF16 = 0, 1
STATUS = {0: "CSA_OK", 1: "CSA_EINVAL", 2: "CSA_EUNSUPPORTED", 3: "CSA_EDEVICE"}

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_sz = ctypes.c_size_t

CSA_LAYER_CSA, CSA_LAYER_HCA = 0, 1


class CsaIn(ctypes.Structure):
    """csa_in: a strided view (base, element strides between sequences and rows)."""
    _fields_ = [("p", ctypes.c_void_p), ("seq_stride", ctypes.c_int64),
                ("row_stride", ctypes.c_int64)]


class CsaOut(ctypes.Structure):
    """csa_out: a strided output view."""
    _fields_ = [("p", ctypes.c_void_p), ("seq_stride", ctypes.c_int64),
                ("row_stride", ctypes.c_int64)]


class LayerDesc(ctypes.Structure):
    """csa_layer_desc: one layer of a stack (kind, m, Nc and device pointers)."""
    _fields_ = [("kind", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("m", ctypes.c_int64), ("Nc", ctypes.c_int64),
                ("q", ctypes.c_void_p), ("ck", ctypes.c_void_p), ("cv", ctypes.c_void_p),
                ("rk", ctypes.c_void_p), ("rv", ctypes.c_void_p), ("q_idx", ctypes.c_void_p),
                ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("topk", ctypes.c_void_p), ("o", ctypes.c_void_p)]


_SIGS = {
    "csa_abi_version": ([], ctypes.c_int),
    "csa_last_error": ([], ctypes.c_char_p),
    "hca_compress": ([ctypes.c_int, _i64, _i64, _i64, _i64, CsaIn, CsaIn, _i64, CsaOut, _p],
                     ctypes.c_int),
    "csa_quantize_mxfp4": ([ctypes.c_int, _i64, _i64, CsaIn, _p, _p, _p], ctypes.c_int),
    "hca_append": ([ctypes.c_int] + [_i64] * 5 + [_p] * 4 + [_i64, _p, _p, _i64,
                   ctypes.POINTER(_i64)] + [_p] * 4 + [_i64, _p], ctypes.c_int),
    "csa_index_topk_workspace": ([_i64] * 9 + [ctypes.POINTER(_sz)], ctypes.c_int),
    "csa_index_topk": ([ctypes.c_int] + [_i64] * 9 + [CsaIn] + [_p] * 4 + [_sz, _p],
                       ctypes.c_int),
    "csa_index_topk_noalloc": ([ctypes.c_int] + [_i64] * 9 + [CsaIn] + [_p] * 3 + [_p],
                               ctypes.c_int),
    "csa_attend_workspace": ([ctypes.c_int] + [_i64] * 6 + [ctypes.POINTER(_sz)], ctypes.c_int),
    "csa_attend": ([ctypes.c_int] + [_i64] * 9 + [ctypes.c_float] + [CsaIn] * 3 + [_p]
                   + [CsaIn] * 2 + [_i64, _i64, CsaOut, _p, _sz, _p], ctypes.c_int),
    "hca_attend_workspace": ([ctypes.c_int] + [_i64] * 8 + [ctypes.POINTER(_sz)], ctypes.c_int),
    "hca_attend": ([ctypes.c_int] + [_i64] * 8 + [ctypes.c_float] + [CsaIn] * 5 + [_i64, _i64]
                   + [CsaOut, _p, _sz, _p], ctypes.c_int),
    "csa_index_attend_workspace": ([ctypes.c_int] + [_i64] * 12 + [ctypes.POINTER(_sz)],
                                   ctypes.c_int),
    "csa_index_attend": ([ctypes.c_int] + [_i64] * 11 + [ctypes.c_float] + [_p] * 8 + [_i64, _i64]
                         + [_p, _p, _i64, _p, _sz, _p, _p], ctypes.c_int),
    "csa_layer_schedule": ([_i64, _p], ctypes.c_int),
    "csa_stack_workspace": ([ctypes.c_int, _i64, _p] + [_i64] * 9 + [ctypes.POINTER(_sz)],
                            ctypes.c_int),
    "csa_stack_attend": ([ctypes.c_int, _i64, _p] + [_i64] * 9 + [ctypes.c_float, _i64, _i64, _p,
                                                                   _sz, _p], ctypes.c_int),
    "csa_quantize_mxfp8": ([ctypes.c_int, _i64, _i64, _p, _p, _p, _p], ctypes.c_int),
    "csa_attend_mxfp8": ([_i64] * 9 + [ctypes.c_float] + [_p] * 8 + [_i64, _i64]
                         + [_p, _p, _sz, _p], ctypes.c_int),
    "hca_attend_mxfp8": ([_i64] * 8 + [ctypes.c_float] + [_p] * 7 + [_i64, _i64]
                         + [_p, _p, _sz, _p], ctypes.c_int),
    "csa_quantize_fp8_rows": ([ctypes.c_int, _i64, _i64, _p, _p, _p, _p], ctypes.c_int),
    "csa_attend_fp8": ([_i64] * 9 + [ctypes.c_float] + [_p] * 10 + [_i64, _i64]
                       + [_p, _p, _sz, _p], ctypes.c_int),
    "hca_attend_fp8": ([_i64] * 8 + [ctypes.c_float] + [_p] * 9 + [_i64, _i64]
                       + [_p, _p, _sz, _p], ctypes.c_int),
}


class CsaError(RuntimeError):
    """A libcsa call returned a status other than CSA_OK."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libcsa.so (once).  Fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CsaError("load", -1, f"{LIB_PATH} is missing; build it with "
                           "`python -m compressed_sparse_attention_04_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise CsaError(name, st, lib().csa_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("this libcsa entry point takes dense row-major tensors")
    return t.data_ptr()


def _rows(t: torch.Tensor, nrow: int):
    """Element strides (between sequences, between rows) of a tensor
    [B, rows, *row] whose last nrow dims form contiguous rows."""
    expect = 1
    for d in range(t.dim() - 1, t.dim() - 1 - nrow, -1):
        if t.shape[d] != 1 and t.stride(d) != expect:
            raise ValueError("libcsa views need each row contiguous")
        expect *= t.shape[d]
    return t.stride(0), t.stride(1)


def _in(t: torch.Tensor, nrow: int = 1) -> CsaIn:
    """A [B, rows, *row] tensor (rows contiguous, any sequence and row
    strides) as a csa_in view."""
    ss, rs = _rows(t, nrow)
    return CsaIn(t.data_ptr(), ss, rs)


def _out(t: torch.Tensor, nrow: int = 1) -> CsaOut:
    ss, rs = _rows(t, nrow)
    return CsaOut(t.data_ptr(), ss, rs)


def _stream(t: torch.Tensor, stream) -> int | None:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    if t.is_cuda:
        return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _keep(t, stream):
    """A tensor this module allocated on the current stream but handed to
    kernels on another stream: tell the caching allocator that the other
    stream uses it, so its memory is not reused before that work is done."""
    if t is None or stream is None or not t.is_cuda:
        return t
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(
        stream, device=t.device)
    if s.cuda_stream != torch.cuda.current_stream(t.device).cuda_stream:
        t.record_stream(s)
    return t


def _workspace(ws, device, query, stream=None):
    """A workspace the caller passed is handed over whole (the library
    checks its size); otherwise one of query() bytes is allocated."""
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    nbytes = query()
    if nbytes == 0:
        return None, 0
    return _keep(torch.empty(nbytes, dtype=torch.uint8, device=device), stream), nbytes


def hca_compress(x: torch.Tensor, gate: torch.Tensor, m: int, out=None, stream=None):
    """Softmax-gated pooling: x [B,T,C], gate [B,T,1|C] -> [B, T//m, C] (any
    views whose rows are contiguous)."""
    B, T, C = x.shape
    if out is None:
        out = _keep(torch.empty((B, T // m, C), dtype=x.dtype, device=x.device), stream)
    _call("hca_compress", _dt(x), B, T, C, m, _in(x), _in(gate), gate.shape[-1], _out(out),
          _stream(x, stream))
    return out


def hca_append(k_new, v_new, gk_new, gv_new, rk, rv, gk_blk, gv_blk, ck, cv, *, m: int, W: int,
               t: int, win_pos0: int, stream=None) -> int:
    """One decode step of cache upkeep: token t [B, C] (gates [B, 1|C]) joins
    the window buffer rk/rv [B, wcap, C] (row r = position win_pos0 + r) and
    the block's gate slots gk_blk/gv_blk [B, m, 1|C]; a completed block is
    pooled into ck/cv [B, nc_cap, C].  Returns the window buffer's first
    position after the call."""
    B, C = k_new.shape
    p0 = ctypes.c_int64(int(win_pos0))
    _call("hca_append", _dt(k_new), B, C, m, W, t, _ptr(k_new), _ptr(v_new), _ptr(gk_new),
          _ptr(gv_new), gk_new.shape[1], _ptr(rk), _ptr(rv), rk.shape[1], ctypes.byref(p0),
          _ptr(gk_blk), _ptr(gv_blk), _ptr(ck), _ptr(cv), ck.shape[1], _stream(k_new, stream))
    return p0.value


def csa_quantize_mxfp4(x: torch.Tensor, codes=None, scales=None, stream=None):
    """MXFP4 encoding of rows of x [..., d]: (codes [..., d/2], scales [..., d/32])."""
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if codes is None:
        codes = _keep(torch.empty(x.shape[:-1] + (d // 2,), dtype=torch.uint8, device=x.device),
                      stream)
    if scales is None:
        scales = _keep(torch.empty(x.shape[:-1] + (d // 32,), dtype=torch.uint8, device=x.device),
                       stream)
    x2 = x.view(rows, d)                  # evenly spaced rows (no copy), else an error
    if d and x2.stride(1) != 1:
        raise ValueError("libcsa views need each row contiguous")
    _call("csa_quantize_mxfp4", _dt(x), rows, d, CsaIn(x.data_ptr(), 0, x2.stride(0)),
          _ptr(codes), _ptr(scales), _stream(x, stream))
    return codes, scales


def csa_index_topk_workspace(B, Tq, HI, dI, Nc, m, W, k, q_pos0) -> int:
    n = _sz(0)
    _call("csa_index_topk_workspace", B, Tq, HI, dI, Nc, m, W, k, q_pos0, ctypes.byref(n))
    return n.value


def csa_index_topk(q_idx: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, *,
                   m: int, W: int, k: int, q_pos0: int, topk=None, ws=None, stream=None):
    """Indexer scores + top-k: q_idx [B,Tq,HI,dI], keys [B,Nc,dI/2]+[B,Nc,dI/32]
    -> topk [B,Tq,k] int32 (ascending, -1 padded)."""
    B, Tq, HI, dI = q_idx.shape
    Nc = k_codes.shape[1]
    ws, wsb = _workspace(ws, q_idx.device,
        lambda: csa_index_topk_workspace(B, Tq, HI, dI, Nc, m, W, k, q_pos0), stream)
    if topk is None:
        topk = _keep(torch.empty((B, Tq, k), dtype=torch.int32, device=q_idx.device), stream)
    _call("csa_index_topk", _dt(q_idx), B, Tq, HI, dI, Nc, m, W, k, q_pos0, _in(q_idx, 2),
          _ptr(k_codes), _ptr(k_scales), _ptr(topk), _ptr(ws), wsb, _stream(q_idx, stream))
    return topk


def csa_index_topk_noalloc(q_idx: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor,
                           *, m: int, W: int, k: int, q_pos0: int, topk=None, stream=None):
    """csa_index_topk with the library's static scratch instead of a workspace
    (the call allocates nothing when topk is given)."""
    B, Tq, HI, dI = q_idx.shape
    Nc = k_codes.shape[1]
    if topk is None:
        topk = _keep(torch.empty((B, Tq, k), dtype=torch.int32, device=q_idx.device), stream)
    _call("csa_index_topk_noalloc", _dt(q_idx), B, Tq, HI, dI, Nc, m, W, k, q_pos0,
          _in(q_idx, 2), _ptr(k_codes), _ptr(k_scales), _ptr(topk), _stream(q_idx, stream))
    return topk


def csa_attend_workspace(dtype: int, B, Tq, H, D, k, W) -> int:
    n = _sz(0)
    _call("csa_attend_workspace", dtype, B, Tq, H, D, k, W, ctypes.byref(n))
    return n.value


def csa_attend(q, ck, cv, topk, rk, rv, *, m: int, W: int, q_pos0: int, raw_pos0: int,
               scale: float = 1.0, out=None, ws=None, stream=None):
    """Attention over the kept compressed entries + raw window -> [B,Tq,H,D]."""
    B, Tq, H, D = q.shape
    Nc = ck.shape[1]
    k = topk.shape[2]
    raw_len = rk.shape[1]
    ws, wsb = _workspace(ws, q.device, lambda: csa_attend_workspace(_dt(q), B, Tq, H, D, k, W),
                          stream)
    if out is None:
        out = _keep(torch.empty_like(q), stream)
    _call("csa_attend", _dt(q), B, Tq, H, D, Nc, m, W, k, q_pos0, scale, _in(q, 2), _in(ck),
          _in(cv), _ptr(topk), _in(rk), _in(rv), raw_pos0, raw_len, _out(out, 2), _ptr(ws),
          wsb, _stream(q, stream))
    return out


def hca_attend_workspace(dtype: int, B, Tq, H, D, Nc, m, W, q_pos0) -> int:
    n = _sz(0)
    _call("hca_attend_workspace", dtype, B, Tq, H, D, Nc, m, W, q_pos0, ctypes.byref(n))
    return n.value


def hca_attend(q, ck, cv, rk, rv, *, m: int, W: int, q_pos0: int, raw_pos0: int,
               scale: float = 1.0, out=None, ws=None, stream=None):
    """Dense attention over every compressed candidate + raw window."""
    B, Tq, H, D = q.shape
    Nc = ck.shape[1]
    raw_len = rk.shape[1]
    ws, wsb = _workspace(ws, q.device,
        lambda: hca_attend_workspace(_dt(q), B, Tq, H, D, Nc, m, W, q_pos0), stream)
    if out is None:
        out = _keep(torch.empty_like(q), stream)
    _call("hca_attend", _dt(q), B, Tq, H, D, Nc, m, W, q_pos0, scale, _in(q, 2), _in(ck),
          _in(cv), _in(rk), _in(rv), raw_pos0, raw_len, _out(out, 2), _ptr(ws), wsb,
          _stream(q, stream))
    return out


def csa_quantize_mxfp8(x: torch.Tensor, codes=None, scales=None, stream=None):
    """MXFP8 (E4M3) encoding of rows of x [..., d]: (codes [..., d], scales [..., d/32])."""
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if codes is None:
        codes = _keep(torch.empty(x.shape, dtype=torch.uint8, device=x.device), stream)
    if scales is None:
        scales = _keep(torch.empty(x.shape[:-1] + (d // 32,), dtype=torch.uint8, device=x.device),
                       stream)
    _call("csa_quantize_mxfp8", _dt(x), rows, d, _ptr(x), _ptr(codes), _ptr(scales),
          _stream(x, stream))
    return codes, scales


def csa_attend_mxfp8(q, ck, cv, ck_scales, cv_scales, topk, rk, rv, *, m: int, W: int,
                     q_pos0: int, raw_pos0: int, scale: float = 1.0, out=None, ws=None,
                     stream=None):
    """csa_attend with MXFP8 compressed entries (codes [B,Nc,128] uint8,
    scales [B,Nc,4] uint8); q, window rows and output bf16."""
    B, Tq, H, D = q.shape
    Nc = ck.shape[1]
    k = topk.shape[2]
    raw_len = rk.shape[1]
    ws, wsb = _workspace(ws, q.device, lambda: csa_attend_workspace(CSA_BF16, B, Tq, H, D, k, W),
                          stream)
    if out is None:
        out = _keep(torch.empty_like(q), stream)
    _call("csa_attend_mxfp8", B, Tq, H, D, Nc, m, W, k, q_pos0, scale, _ptr(q), _ptr(ck),
          _ptr(cv), _ptr(ck_scales), _ptr(cv_scales), _ptr(topk), _ptr(rk), _ptr(rv), raw_pos0,
          raw_len, _ptr(out), _ptr(ws), wsb, _stream(q, stream))
    return out


def hca_attend_mxfp8(q, ck, cv, ck_scales, cv_scales, rk, rv, *, m: int, W: int, q_pos0: int,
                     raw_pos0: int, scale: float = 1.0, out=None, ws=None, stream=None):
    """hca_attend with MXFP8 compressed entries."""
    B, Tq, H, D = q.shape
    Nc = ck.shape[1]
    raw_len = rk.shape[1]
    ws, wsb = _workspace(ws, q.device,
        lambda: hca_attend_workspace(CSA_BF16, B, Tq, H, D, Nc, m, W, q_pos0), stream)
    if out is None:
        out = _keep(torch.empty_like(q), stream)
    _call("hca_attend_mxfp8", B, Tq, H, D, Nc, m, W, q_pos0, scale, _ptr(q), _ptr(ck), _ptr(cv),
          _ptr(ck_scales), _ptr(cv_scales), _ptr(rk), _ptr(rv), raw_pos0, raw_len, _ptr(out),
          _ptr(ws), wsb, _stream(q, stream))
    return out


def csa_layer_schedule(n_layers: int) -> list:
    """Layer kinds of an n-layer stack (CSA_LAYER_CSA / CSA_LAYER_HCA)."""
    kinds = (ctypes.c_int32 * max(1, n_layers))()
    _call("csa_layer_schedule", n_layers, ctypes.cast(kinds, ctypes.c_void_p))
    return list(kinds)[:n_layers]


def _layer_array(layers):
    """layers: dicts with kind, m and the layer's tensors (q, ck, cv, rk, rv, o;
    CSA also q_idx, k_codes, k_scales, topk)."""
    arr = (LayerDesc * max(1, len(layers)))()
    for i, L in enumerate(layers):
        d = arr[i]
        d.kind, d.m, d.Nc = int(L["kind"]), int(L["m"]), int(L["ck"].shape[1])
        for f in ("q", "ck", "cv", "rk", "rv", "q_idx", "k_codes", "k_scales", "topk", "o"):
            setattr(d, f, _ptr(L.get(f)))
    return arr


def csa_stack_workspace(dtype: int, layers, B, Tq, H, D, HI, dI, W, k, q_pos0) -> int:
    n = _sz(0)
    arr = _layer_array(layers)
    _call("csa_stack_workspace", dtype, len(layers), ctypes.cast(arr, ctypes.c_void_p), B, Tq, H,
          D, HI, dI, W, k, q_pos0, ctypes.byref(n))
    return n.value


def csa_stack_attend(layers, *, W: int, k: int, q_pos0: int, raw_pos0: int, scale: float = 1.0,
                     HI: int = 4, dI: int = 64, ws=None, stream=None):
    """Run every layer of the stack in order (see csa_stack_attend in csa.h);
    each layer's output goes to its "o" tensor (and a CSA layer's selection
    to its "topk")."""
    q = layers[0]["q"]
    B, Tq, H, D = q.shape
    raw_len = layers[0]["rk"].shape[1]
    arr = _layer_array(layers)
    ws, wsb = _workspace(ws, q.device,
        lambda: csa_stack_workspace(_dt(q), layers, B, Tq, H, D, HI, dI, W, k, q_pos0), stream)
    _call("csa_stack_attend", _dt(q), len(layers), ctypes.cast(arr, ctypes.c_void_p), B, Tq, H, D,
          HI, dI, W, k, q_pos0, scale, raw_pos0, raw_len, _ptr(ws), wsb, _stream(q, stream))


_aux_streams = {}


def csa_index_attend_workspace(dtype: int, B, Tq, H, D, HI, dI, Nc, m, W, k, q_pos0,
                               n_chunks) -> int:
    n = _sz(0)
    _call("csa_index_attend_workspace", dtype, B, Tq, H, D, HI, dI, Nc, m, W, k, q_pos0,
          n_chunks, ctypes.byref(n))
    return n.value


def csa_index_attend(q, q_idx, k_codes, k_scales, ck, cv, rk, rv, *, m: int, W: int, k: int,
                     q_pos0: int, raw_pos0: int, n_chunks: int = 8, scale: float = 1.0,
                     topk=None, out=None, ws=None, stream=None, aux_stream=None):
    """csa_index_topk + csa_attend as one pipeline over n_chunks query slices
    (selection on aux_stream, attention on stream).  Returns (topk, out)."""
    B, Tq, H, D = q.shape
    HI, dI = q_idx.shape[2], q_idx.shape[3]
    Nc = ck.shape[1]
    raw_len = rk.shape[1]
    if aux_stream is None:
        dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
        if dev not in _aux_streams:
            _aux_streams[dev] = torch.cuda.Stream(device=dev)
        aux_stream = _aux_streams[dev]
    own_ws = ws is None
    ws, wsb = _workspace(ws, q.device,
        lambda: csa_index_attend_workspace(_dt(q), B, Tq, H, D, HI, dI, Nc, m, W, k, q_pos0,
                                        n_chunks), stream)
    if own_ws:
        _keep(ws, aux_stream)            # the selection slices run on aux_stream
    if topk is None:
        topk = _keep(_keep(torch.empty((B, Tq, k), dtype=torch.int32, device=q.device), stream),
                     aux_stream)
    if out is None:
        out = _keep(torch.empty_like(q), stream)
    _call("csa_index_attend", _dt(q), B, Tq, H, D, HI, dI, Nc, m, W, k, q_pos0, scale, _ptr(q),
          _ptr(q_idx), _ptr(k_codes), _ptr(k_scales), _ptr(ck), _ptr(cv), _ptr(rk), _ptr(rv),
          raw_pos0, raw_len, _ptr(topk), _ptr(out), n_chunks, _ptr(ws), wsb, _stream(q, stream),
          _stream(q, aux_stream))
    return topk, out


def csa_quantize_fp8_rows(x: torch.Tensor, codes=None, scales=None, stream=None):
    """E4M3 encoding of rows of x [..., d] with one scale per row: (codes
    [..., d] uint8, scales [...] int32 words holding the fp32 bits of 2^e)."""
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if codes is None:
        codes = _keep(torch.empty(x.shape, dtype=torch.uint8, device=x.device), stream)
    if scales is None:
        scales = _keep(torch.empty(x.shape[:-1], dtype=torch.int32, device=x.device), stream)
    _call("csa_quantize_fp8_rows", _dt(x), rows, d, _ptr(x), _ptr(codes), _ptr(scales),
          _stream(x, stream))
    return codes, scales


def csa_attend_fp8(q, ck, cv, ck_scales, cv_scales, topk, rk, rv, rk_scales, rv_scales, *,
                   m: int, W: int, q_pos0: int, raw_pos0: int, scale: float = 1.0, out=None,
                   ws=None, stream=None):
    """csa_attend with FP8 arithmetic: compressed and window rows as FP8 rows
    (codes [B,N,128] uint8, scale words [B,N] int32); q and output bf16."""
    B, Tq, H, D = q.shape
    Nc = ck.shape[1]
    k = topk.shape[2]
    raw_len = rk.shape[1]
    ws, wsb = _workspace(ws, q.device, lambda: csa_attend_workspace(CSA_BF16, B, Tq, H, D, k, W),
                          stream)
    if out is None:
        out = _keep(torch.empty_like(q), stream)
    _call("csa_attend_fp8", B, Tq, H, D, Nc, m, W, k, q_pos0, scale, _ptr(q), _ptr(ck),
          _ptr(cv), _ptr(ck_scales), _ptr(cv_scales), _ptr(topk), _ptr(rk), _ptr(rv),
          _ptr(rk_scales), _ptr(rv_scales), raw_pos0, raw_len, _ptr(out), _ptr(ws), wsb,
          _stream(q, stream))
    return out


def hca_attend_fp8(q, ck, cv, ck_scales, cv_scales, rk, rv, rk_scales, rv_scales, *, m: int,
                   W: int, q_pos0: int, raw_pos0: int, scale: float = 1.0, out=None, ws=None,
                   stream=None):
    """hca_attend with FP8 arithmetic (see csa_attend_fp8)."""
    B, Tq, H, D = q.shape
    Nc = ck.shape[1]
    raw_len = rk.shape[1]
    ws, wsb = _workspace(ws, q.device,
        lambda: hca_attend_workspace(CSA_BF16, B, Tq, H, D, Nc, m, W, q_pos0), stream)
    if out is None:
        out = _keep(torch.empty_like(q), stream)
    _call("hca_attend_fp8", B, Tq, H, D, Nc, m, W, q_pos0, scale, _ptr(q), _ptr(ck), _ptr(cv),
          _ptr(ck_scales), _ptr(cv_scales), _ptr(rk), _ptr(rv), _ptr(rk_scales),
          _ptr(rv_scales), raw_pos0, raw_len, _ptr(out), _ptr(ws), wsb, _stream(q, stream))
    return out
