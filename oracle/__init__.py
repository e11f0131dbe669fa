"""CPU oracle for compressed sparse attention (CSA) and heavily compressed
attention (HCA): a plain fp64 C implementation (``csa_oracle.c``) behind a
ctypes wrapper that takes and returns numpy arrays.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product library
never loads it, and it shares no code with the GPU path.

Every function states the passage it follows; the readings taken where the
pages are silent are spelled out in ``csa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile ``csa_oracle.c`` with gcc (OpenMP over independent rows)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_abi_version.restype = ctypes.c_int
        L.oracle_compress.argtypes = [_i64, _i64, _i64, _i64, _ptr, _ptr, _i64, _ptr]
        L.oracle_quant_mxfp4.argtypes = [_i64, _i64, _ptr, _ptr, _ptr]
        L.oracle_mxfp4_value.argtypes = [ctypes.c_int, ctypes.c_int]
        L.oracle_mxfp4_value.restype = ctypes.c_double
        L.oracle_quant_mxfp8.argtypes = [_i64, _i64, _ptr, _ptr, _ptr]
        L.oracle_quant_fp8_rows.argtypes = [_i64, _i64, _ptr, _ptr, _ptr]
        L.oracle_mxfp8_value.argtypes = [ctypes.c_int, ctypes.c_int]
        L.oracle_mxfp8_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_int]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_n_cand.argtypes = [_i64, _i64, _i64]
        L.oracle_n_cand.restype = _i64
        L.oracle_index_scores.argtypes = [_i64] * 7 + [_ptr] * 7
        L.oracle_select_topk.argtypes = [_i64] * 6 + [_ptr] * 3
        L.oracle_index_topk.argtypes = [_i64] * 8 + [_ptr] * 7
        L.oracle_attend.argtypes = ([_i64] * 8 + [_ptr, ctypes.c_double] + [_ptr] * 6
                                    + [_i64, _i64, _ptr])
        L.oracle_attend_stats.argtypes = ([_i64] * 8 + [_ptr, ctypes.c_double] + [_ptr] * 6
                                          + [_i64, _i64, _ptr, _ptr, _ptr])
        for f in ("oracle_compress", "oracle_quant_mxfp4", "oracle_quant_mxfp8",
                  "oracle_quant_fp8_rows", "oracle_index_scores", "oracle_select_topk",
                  "oracle_index_topk", "oracle_attend", "oracle_attend_stats"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def compress(x, gate, m: int) -> np.ndarray:
    """Softmax-gated pooling of m adjacent rows (jiwasawa.github.io post,
    CSA token-level compression; studioglobal.ai answer, CSA bullet).
    x [B,T,C], gate [B,T,1] or [B,T,C] -> [B, T//m, C] (fp64)."""
    if m <= 0:
        raise ValueError("oracle compress: m must be positive")
    x = _f64(x)
    gate = _f64(gate)
    B, T, C = x.shape
    gc = gate.shape[2]
    out = np.zeros((B, T // m, C), np.float64)
    _check(lib().oracle_compress(B, T, C, m, _p(x), _p(gate), gc, _p(out)), "compress")
    return out


def quant_mxfp4(x):
    """MXFP4 encoding of rows of x [..., d] (d % 32 == 0): returns
    (codes [..., d/2] uint8, scales [..., d/32] uint8)."""
    x = _f64(x)
    shape = x.shape
    d = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    codes = np.zeros(shape[:-1] + (d // 2,), np.uint8)
    scales = np.zeros(shape[:-1] + (d // 32,), np.uint8)
    _check(lib().oracle_quant_mxfp4(rows, d, _p(x), _p(codes), _p(scales)), "quant_mxfp4")
    return codes, scales


def mxfp4_value(code: int, scale: int) -> float:
    return lib().oracle_mxfp4_value(int(code), int(scale))


def quant_mxfp8(x):
    """MXFP8 (E4M3) encoding of rows of x [..., d] (d % 32 == 0), the storage
    of the compressed KV entries (ai-papers.net article, hybrid attention
    section: most KV entries in FP8): returns (codes [..., d] uint8,
    scales [..., d/32] uint8)."""
    x = _f64(x)
    shape = x.shape
    d = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    codes = np.zeros(shape, np.uint8)
    scales = np.zeros(shape[:-1] + (d // 32,), np.uint8)
    _check(lib().oracle_quant_mxfp8(rows, d, _p(x), _p(codes), _p(scales)), "quant_mxfp8")
    return codes, scales


def quant_fp8_rows(x):
    """E4M3 encoding of rows of x [..., d] (d % 32 == 0) with ONE scale
    exponent per row (reading R13d: the FP8 attention arithmetic; the
    exponent rule of the MXFP8 runs applied to the whole row).  Returns
    (codes [..., d] uint8, scales [..., d/32] uint8), the row's exponent
    repeated in each of its d/32 scale bytes (a valid MXFP8 row)."""
    x = _f64(x)
    shape = x.shape
    d = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    codes = np.zeros(shape, np.uint8)
    scales = np.zeros(shape[:-1] + (d // 32,), np.uint8)
    _check(lib().oracle_quant_fp8_rows(rows, d, _p(x), _p(codes), _p(scales)), "quant_fp8_rows")
    return codes, scales


def mxfp8_value(code: int, scale: int) -> float:
    return lib().oracle_mxfp8_value(int(code), int(scale))


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def dequant_mxfp8(codes, scales) -> np.ndarray:
    """Exact values (fp64) of MXFP8 rows: codes [..., d], scales [..., d/32]."""
    c = np.ascontiguousarray(codes, np.uint8)
    s = np.ascontiguousarray(scales, np.uint8)
    mag = np.array([e4m3_value(v) for v in range(128)], np.float64)
    val = mag[c & 0x7F] * np.where(c & 0x80, -1.0, 1.0)
    sc = np.ldexp(1.0, s.astype(np.int64) - 127)
    return val * np.repeat(sc, 32, axis=-1)


def n_cand(t: int, m: int, W: int) -> int:
    """Number of compressed candidates of a query at position t."""
    return int(lib().oracle_n_cand(int(t), int(m), int(W)))


def index_scores(q_codes, q_scales, k_codes, k_scales, q_pos, m: int, W: int):
    """Exact indexer scores [B,Tq,Nc] (-1 for non-candidates) and the fp32
    exactness flag.  q_codes [B,Tq,HI,dI/2], k_codes [B,Nc,dI/2]."""
    qc = np.ascontiguousarray(q_codes, np.uint8)
    qs = np.ascontiguousarray(q_scales, np.uint8)
    kc = np.ascontiguousarray(k_codes, np.uint8)
    ks = np.ascontiguousarray(k_scales, np.uint8)
    qp = np.ascontiguousarray(q_pos, np.int64)
    B, Tq, HI, half = qc.shape
    Nc = kc.shape[1]
    dI = half * 2
    scores = np.zeros((B, Tq, Nc), np.float32)
    exact = ctypes.c_int(0)
    _check(lib().oracle_index_scores(B, Tq, HI, dI, Nc, m, W, _p(qp), _p(qc), _p(qs),
                                     _p(kc), _p(ks), _p(scores),
                                     ctypes.cast(ctypes.pointer(exact), ctypes.c_void_p)),
           "index_scores")
    return scores, bool(exact.value)


def select_topk(scores, q_pos, m: int, W: int, k: int) -> np.ndarray:
    """Top-k of each row of scores [B,Tq,Nc] under (score desc, index asc),
    ascending indices, -1 padded."""
    s = np.ascontiguousarray(scores, np.float32)
    qp = np.ascontiguousarray(q_pos, np.int64)
    B, Tq, Nc = s.shape
    out = np.zeros((B, Tq, k), np.int32)
    _check(lib().oracle_select_topk(B, Tq, Nc, m, W, k, _p(qp), _p(s), _p(out)), "select_topk")
    return out


def index_topk(q_idx, k_codes, k_scales, q_pos, m: int, W: int, k: int):
    """Quantise q_idx [B,Tq,HI,dI] to MXFP4, score every candidate, keep the
    top k.  Returns (topk [B,Tq,k] int32, exact flag)."""
    qc, qs = quant_mxfp4(q_idx)
    kc = np.ascontiguousarray(k_codes, np.uint8)
    ks = np.ascontiguousarray(k_scales, np.uint8)
    qp = np.ascontiguousarray(q_pos, np.int64)
    B, Tq, HI, dI = np.asarray(q_idx).shape
    Nc = kc.shape[1]
    out = np.zeros((B, Tq, k), np.int32)
    exact = ctypes.c_int(0)
    _check(lib().oracle_index_topk(B, Tq, HI, dI, Nc, m, W, k, _p(qp), _p(qc), _p(qs),
                                   _p(kc), _p(ks), _p(out),
                                   ctypes.cast(ctypes.pointer(exact), ctypes.c_void_p)),
           "index_topk")
    return out, bool(exact.value)


def _attend(q, ck, cv, topk, rk, rv, raw_pos0: int, q_pos, m: int, W: int, scale: float,
            stats: bool):
    q = _f64(q)
    ck = _f64(ck)
    cv = _f64(cv)
    rk = _f64(rk)
    rv = _f64(rv)
    qp = np.ascontiguousarray(q_pos, np.int64)
    B, Tq, H, D = q.shape
    Nc = ck.shape[1]
    raw_len = rk.shape[1]
    if topk is None:
        k = 0
        tk = None
    else:
        tk = np.ascontiguousarray(topk, np.int32)
        k = tk.shape[2]
    o = np.zeros((B, Tq, H, D), np.float64)
    am = np.zeros((B, Tq, H, D), np.float64) if stats else None
    rm = np.zeros((B, Tq, H, D), np.float64) if stats else None
    _check(lib().oracle_attend_stats(B, Tq, H, D, Nc, m, W, k, _p(qp), scale, _p(q), _p(ck),
                                     _p(cv), None if tk is None else _p(tk), _p(rk), _p(rv),
                                     raw_pos0, raw_len, _p(o),
                                     None if am is None else _p(am),
                                     None if rm is None else _p(rm)), "attend")
    return (o, am, rm) if stats else o


def attend(q, ck, cv, topk, rk, rv, raw_pos0: int, q_pos, m: int, W: int,
           scale: float = 1.0) -> np.ndarray:
    """One softmax over the selected (topk given: CSA) or all (topk None:
    HCA) compressed candidates joined with the raw window w0..t
    (jiwasawa.github.io post, CSA "Shared Key-Value MQA" and HCA parts, SWA
    branch).  q [B,Tq,H,D], ck/cv [B,Nc,D], rk/rv [B,raw_len,D] -> o (fp64)."""
    return _attend(q, ck, cv, topk, rk, rv, raw_pos0, q_pos, m, W, scale, False)


def attend_stats(q, ck, cv, topk, rk, rv, raw_pos0: int, q_pos, m: int, W: int,
                 scale: float = 1.0):
    """attend, plus per output element the softmax-weighted means
    amean = sum p|v| / sum p and rms = sqrt(sum p^2 v^2) / sum p over the
    key list: (o, amean, rms), each [B,Tq,H,D] fp64."""
    return _attend(q, ck, cv, topk, rk, rv, raw_pos0, q_pos, m, W, scale, True)


def attend_fp8(q, ck, ck_scales, cv, cv_scales, topk, rk, rk_scales, rv, rv_scales,
               raw_pos0: int, q_pos, m: int, W: int, scale: float = 1.0):
    """Attention with FP8 arithmetic (reading R13d; ai-papers.net article,
    hybrid attention section: most KV entries in FP8).  Keys and values of
    the compressed entries and of the raw window are FP8 rows (codes and
    scales as quant_fp8_rows writes them, decoded exactly); each query
    head's row of q [B,Tq,H,D] is encoded the same way (one exponent per
    head row) and decoded; then one exact softmax over the key list as in
    attend.  Returns (o, amean, rms) as attend_stats."""
    qc, qs = quant_fp8_rows(q)
    return attend_stats(dequant_mxfp8(qc, qs), dequant_mxfp8(ck, ck_scales),
                        dequant_mxfp8(cv, cv_scales), topk, dequant_mxfp8(rk, rk_scales),
                        dequant_mxfp8(rv, rv_scales), raw_pos0, q_pos, m, W, scale)


def set_threads(n: int) -> None:
    """Host threads that the oracle's parallel row loops use from now on (the
    OpenMP runtime the oracle is linked against; no arithmetic changes)."""
    lib()
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
