"""C-ABI contract of libcsa.so on a host without a GPU: the library loads,
exports every entry point include/csa.h declares, sizes workspaces, and
rejects invalid arguments with CSA_EINVAL / CSA_EUNSUPPORTED and a message
before anything reaches the device."""
import ctypes
import os
import re

import pytest

from compressed_sparse_attention_04_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

EINVAL, EUNSUP = 1, 2
P = ctypes.c_void_p(0x1000)          # aligned non-null placeholder; never dereferenced


def V(row, rows=1 << 20, p=0x1000, ss=None, rs=None, out=False):
    """A view placeholder (never dereferenced): rows of `row` elements,
    dense unless strides are given."""
    rs = row if rs is None else rs
    ss = rows * rs if ss is None else ss
    return (binding.CsaOut if out else binding.CsaIn)(p, ss, rs)


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:csa_status|int|const char \*)\s*(\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from compressed_sparse_attention_04_amd import build
        build.build()
    return binding.lib()


def test_exports_every_declared_symbol(L):
    names = declared()
    assert {"hca_compress", "csa_index_topk", "csa_attend", "hca_attend",
            "csa_quantize_mxfp4", "hca_append", "csa_quantize_mxfp8", "csa_attend_mxfp8",
            "hca_attend_mxfp8", "csa_layer_schedule", "csa_stack_workspace",
            "csa_stack_attend", "csa_index_attend_workspace", "csa_index_attend",
            "csa_quantize_fp8_rows", "csa_attend_fp8", "hca_attend_fp8"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(binding._SIGS), "binding and header disagree"


def test_version(L):
    want = int(re.search(r"#define CSA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert L.csa_abi_version() == want == 8


def err(L):
    return L.csa_last_error().decode()


def test_compress_rejects(L):
    x, g, o = V(8, 8), V(1, 8), V(8, 2, out=True)
    assert L.hca_compress(7, 1, 8, 8, 4, x, g, 1, o, None) == EINVAL
    assert "dtype" in err(L)
    assert L.hca_compress(1, 1, 8, 12, 4, V(12, 8), g, 1, V(12, 2, out=True), None) == EINVAL
    assert L.hca_compress(1, 1, 8, 8, 0, x, g, 1, o, None) == EINVAL      # m
    assert L.hca_compress(1, 1, 8, 8, 4, x, g, 3, o, None) == EINVAL      # gate channels
    assert L.hca_compress(1, 1, 8, 8, 4, V(8, 8, p=0), g, 1, o, None) == EINVAL   # null
    assert "null" in err(L)
    assert L.hca_compress(1, 1, 8, 8, 4, V(8, 8, p=0x1002), g, 1, o, None) == EINVAL
    assert "aligned" in err(L)


def test_views_rejected(L):
    """Strided views: rows that overlap, negative or misaligned strides, and
    output sequences that overlap are refused before any launch."""
    g = V(1, 64)
    f = lambda x, o, B=1: L.hca_compress(1, B, 64, 128, 4, x, V(1, 64, ss=64), 1, o, None)
    assert f(V(128, 64, rs=64), V(128, 16, out=True)) == EINVAL            # rows overlap
    assert "row stride" in err(L)
    assert f(V(128, 64, rs=-128), V(128, 16, out=True)) == EINVAL          # negative
    assert f(V(128, 64, rs=132), V(128, 16, out=True)) == EINVAL           # 264-byte rows
    assert "aligned" in err(L)
    assert f(V(128, 64, ss=9000 * 128), V(128, 16, ss=8 * 128, out=True), B=2) == EINVAL
    assert "overlap" in err(L)                                            # out sequences
    # a window of raw rows and query rows taken from larger buffers pass the
    # view checks (the raw-position check, made after them, is what fails)
    q, ck = V(128 * 128, 4, ss=100 * 128 * 128), V(128, 300, rs=256)
    st = L.hca_attend(1, 2, 4, 128, 128, 300, 4, 128, 1196, 1.0, q, ck, ck, V(128, 128, rs=512),
                      V(128, 128, rs=512), 1073, 127, V(128 * 128, 4, out=True), None, 0, None)
    assert st == EINVAL and "raw rows" in err(L)
    # key rows spanning more than 2 GiB in one sequence
    st = L.hca_attend(1, 1, 1, 128, 128, 300, 4, 128, 1199, 1.0, V(128 * 128, 1), V(128, 300,
                      rs=1 << 23), V(128, 300), V(128, 128), V(128, 128), 1072, 128,
                      V(128 * 128, 1, out=True), None, 0, None)
    assert st == EUNSUP and "2 GiB" in err(L)


def test_append_rejects(L):
    def call(dt=1, B=1, C=128, m=4, W=128, t=10, gc=128, wcap=256, p0=0, nc_cap=64, kn=P):
        pos = ctypes.c_int64(p0)
        st = L.hca_append(dt, B, C, m, W, t, kn, P, P, P, gc, P, P, wcap, ctypes.byref(pos), P,
                          P, P, P, nc_cap, None)
        return st, pos.value
    assert call(dt=7)[0] == EINVAL and "dtype" in err(L)
    assert call(C=12)[0] == EINVAL                        # C % 8
    assert call(m=0)[0] == EINVAL and call(m=200)[0] == EINVAL   # 1 <= m <= W
    assert call(wcap=200)[0] == EINVAL                    # wcap >= 2W
    assert call(gc=3)[0] == EINVAL                        # gate channels
    assert call(t=300, p0=200)[0] == EINVAL               # buffer lacks positions 173 .. 199
    assert "window buffer" in err(L)
    assert call(t=600, p0=300)[0] == EINVAL               # past the buffer's capacity
    assert call(t=5, p0=1)[0] == EINVAL                   # lacks position 0
    assert call(t=399, p0=200, nc_cap=99)[0] == EINVAL    # entry 99 does not fit
    assert "nc_cap" in err(L)
    assert call(kn=None)[0] == EINVAL and "null" in err(L)
    assert call(kn=ctypes.c_void_p(0x1002))[0] == EINVAL and "aligned" in err(L)
    st, pos = call(t=300, p0=200)
    assert st == EINVAL and pos == 200                    # unchanged on an error


def test_quantize_rejects(L):
    assert L.csa_quantize_mxfp4(1, 4, 48, V(48, 4), P, P, None) == EINVAL
    assert L.csa_quantize_mxfp4(1, 4, 64, V(64, 4), None, P, None) == EINVAL
    assert L.csa_quantize_mxfp4(1, 4, 64, V(64, 4, rs=32), P, P, None) == EINVAL   # overlap


def test_mxfp8_rejects(L):
    assert L.csa_quantize_mxfp8(1, 4, 48, P, P, P, None) == EINVAL            # d % 32
    assert L.csa_quantize_mxfp8(1, 4, 64, P, None, P, None) == EINVAL         # null
    assert L.csa_quantize_mxfp8(5, 4, 64, P, P, P, None) == EINVAL            # dtype
    S = ctypes.c_void_p(0x1004)                        # 4-byte aligned scales are fine
    def hca(D=128, H=128, cks=S, q=P):
        return L.hca_attend_mxfp8(1, 1, H, D, 300, 4, 128, 1199, 1.0, q, P, P, cks, S, P, P,
                                  1072, 128, P, None, 0, None)
    assert hca(D=64) == EUNSUP and "D = 128" in err(L)
    assert hca(H=96) == EUNSUP
    assert hca(cks=ctypes.c_void_p(0x1002)) == EINVAL and "4-byte" in err(L)
    assert hca(q=None) == EINVAL and "null" in err(L)
    st = L.csa_attend_mxfp8(1, 1, 128, 128, 300, 4, 128, 16, 1199, 1.0, P, P, P, S, S, None, P,
                            P, 1072, 128, P, None, 0, None)
    assert st == EINVAL and "null" in err(L)                # topk
    st = L.csa_attend_mxfp8(1, 1, 128, 128, 300, 4, 128, 16, 1199, 1.0, P, P, P, S, S, P, P, P,
                            1073, 127, P, None, 0, None)
    assert st == EINVAL and "raw rows" in err(L)


def test_fp8_rejects(L):
    assert L.csa_quantize_fp8_rows(1, 4, 96, P, P, P, None) == EUNSUP          # d
    assert L.csa_quantize_fp8_rows(1, 4, 64, P, None, P, None) == EINVAL       # null
    assert L.csa_quantize_fp8_rows(5, 4, 64, P, P, P, None) == EINVAL          # dtype
    assert L.csa_quantize_fp8_rows(1, 4, 64, ctypes.c_void_p(0x1008), P, P, None) == EINVAL
    assert L.csa_quantize_fp8_rows(1, 0, 64, None, None, None, None) == 0      # nothing to do
    S = ctypes.c_void_p(0x1004)                        # 4-byte aligned scales are fine
    def hca(D=128, H=128, cks=S, rvs=S, q=P, p0=1072, rl=128):
        return L.hca_attend_fp8(1, 1, H, D, 300, 4, 128, 1199, 1.0, q, P, P, cks, S, P, P, S,
                                rvs, p0, rl, P, None, 0, None)
    assert hca(D=64) == EUNSUP and "D = 128" in err(L)
    assert hca(H=96) == EUNSUP
    assert hca(cks=ctypes.c_void_p(0x1002)) == EINVAL and "4-byte" in err(L)
    assert hca(rvs=None) == EINVAL and "null" in err(L)
    assert hca(q=None) == EINVAL and "null" in err(L)
    assert hca(p0=1073, rl=127) == EINVAL and "raw rows" in err(L)
    def csa(topk=P, k=16):
        return L.csa_attend_fp8(1, 1, 128, 128, 300, 4, 128, k, 1199, 1.0, P, P, P, S, S, topk,
                                P, P, S, S, 1072, 128, P, None, 0, None)
    assert csa(topk=None) == EINVAL and "null" in err(L)
    assert csa(k=0) == EINVAL and csa(k=4096) == EINVAL
    # the split plan of a decode row needs a workspace
    st = L.hca_attend_fp8(4, 1, 128, 128, 8191, 128, 128, 1048575, 1.0, P, P, P, S, S, P, P, S,
                          S, 1048448, 128, P, None, 0, None)
    assert st == EINVAL and "workspace" in err(L)


def test_index_attend_rejects(L):
    n = ctypes.c_size_t(0)
    ws = lambda nch, Nc=600, k=512: L.csa_index_attend_workspace(1, 1, 100, 128, 128, 4, 64, Nc,
                                                                  4, 128, k, 2000, nch,
                                                                  ctypes.byref(n))
    assert ws(0) == EINVAL and "n_chunks" in err(L)
    assert ws(65) == EINVAL
    assert ws(4, Nc=100) == EINVAL and "candidates" in err(L)
    assert ws(4, k=4096) == EINVAL
    assert ws(4) == 0

    def call(nch=4, raw_pos0=0, topk=P, wsb=1 << 30):
        return L.csa_index_attend(1, 1, 100, 128, 128, 4, 64, 600, 4, 128, 512, 2000, 1.0, P, P,
                                  P, P, P, P, P, P, raw_pos0, 2100, topk, P, nch, P, wsb, None,
                                  None)
    assert call(nch=0) == EINVAL
    assert call(topk=None) == EINVAL and "null" in err(L)
    assert call(raw_pos0=1900) == EINVAL and "raw rows" in err(L)
    assert n.value > 0                                    # 25-row slices split their keys
    assert call(wsb=n.value - 1) == EINVAL and "workspace" in err(L)


def test_layer_schedule():
    kinds = binding.csa_layer_schedule(61)
    H, C = binding.CSA_LAYER_HCA, binding.CSA_LAYER_CSA
    assert kinds[:4] == [H, H, C, H] and kinds[-1] == C
    assert kinds.count(C) == 30 and kinds.count(H) == 31
    assert all(kinds[l] == (C if l % 2 == 0 else H) for l in range(2, 61))
    assert binding.csa_layer_schedule(0) == []


def test_stack_rejects_before_any_launch(L):
    # a valid HCA layer, then a CSA layer whose cache is too short: nothing may
    # launch (null stream, fake device pointers), and the error names layer 1
    arr = (binding.LayerDesc * 2)()
    for d in arr:
        d.q = d.ck = d.cv = d.rk = d.rv = d.o = 0x1000
        d.q_idx = d.k_codes = d.k_scales = d.topk = 0x1000
    arr[0].kind, arr[0].m, arr[0].Nc = binding.CSA_LAYER_HCA, 128, 16
    arr[1].kind, arr[1].m, arr[1].Nc = binding.CSA_LAYER_CSA, 4, 100
    args = (1, 2, ctypes.cast(arr, ctypes.c_void_p), 1, 1, 128, 128, 4, 64, 128, 512, 2047)
    n = ctypes.c_size_t(0)
    assert L.csa_stack_workspace(*args, ctypes.byref(n)) == EINVAL
    assert err(L).startswith("layer 1:") and "candidates" in err(L)
    assert L.csa_stack_attend(*args, 1.0, 1920, 128, None, 0, None) == EINVAL
    assert "layer 1" in err(L)
    arr[1].Nc = 600                                    # valid now; layer 0 loses its window
    assert L.csa_stack_workspace(*args, ctypes.byref(n)) == 0
    assert L.csa_stack_attend(*args, 1.0, 1921, 128, None, 0, None) == EINVAL
    assert "csa_stack_attend: layer 0: hca_attend" in err(L)
    arr[0].kind = 7
    assert L.csa_stack_workspace(*args, ctypes.byref(n)) == EINVAL and "unknown kind" in err(L)


def ws_index(L, *a):
    n = ctypes.c_size_t(0)
    st = L.csa_index_topk_workspace(*a, ctypes.byref(n))
    return st, n.value


def test_index_workspace_and_rejects(L):
    # decode rows over 262,112 candidates, per row: 64 chunks of 4096, each
    # with a list of 32 (key, index) pairs (4 x 512 x 4096 / 262112 rounded up
    # to a power of two) and one (count, threshold) pair; no score array
    st, n = ws_index(L, 16, 1, 4, 64, 262144, 4, 128, 512, (1 << 20) - 1)
    assert st == 0 and n == 16 * 64 * (32 + 1) * 8
    # k = 2048: 128 pairs per chunk
    st, n = ws_index(L, 16, 1, 4, 64, 262144, 4, 128, 2048, (1 << 20) - 1)
    assert st == 0 and n == 16 * 64 * (128 + 1) * 8
    # 8 rows: chunks of 1024 (256 of them), 32 pairs each
    st, n = ws_index(L, 2, 8, 4, 64, 262144, 4, 128, 512, (1 << 20) - 8)
    assert st == 0 and n == 16 * 256 * (32 + 1) * 8
    # the streaming path (<= 32768 candidates) needs no workspace
    st, n = ws_index(L, 1, 16, 2, 32, 256, 4, 128, 16, 1008)
    assert st == 0 and n == 0
    st, n = ws_index(L, 1, 32768, 4, 64, 8192, 4, 128, 512, 0)
    assert st == 0 and n == 0
    # > 8 rows over > 32768 candidates: chunk lists of (key, index) pairs,
    # 9 chunks of 4096 for 34,966 candidates
    st, n = ws_index(L, 1, 10, 4, 64, 35000, 4, 128, 512, 139990)
    assert st == 0 and n == 10 * 9 * 512 * 8
    assert ws_index(L, 1, 16, 3, 32, 256, 4, 128, 16, 1008)[0] == EUNSUP      # HI
    assert ws_index(L, 1, 16, 2, 48, 256, 4, 128, 16, 1008)[0] == EUNSUP      # dI
    assert ws_index(L, 1, 16, 2, 32, 256, 4, 128, 4096, 1008)[0] == EINVAL    # k
    assert ws_index(L, 1, 16, 2, 32, 200, 4, 128, 16, 1008)[0] == EINVAL      # Nc short
    assert "candidates" in err(L)
    # a workspace that is too small is refused before launch
    st = L.csa_index_topk(1, 16, 1, 4, 64, 262144, 4, 128, 512, (1 << 20) - 1,
                          V(256, 1), P, P, P, P, 1024, None)
    assert st == EINVAL and "workspace" in err(L)


def test_attend_workspace_and_rejects(L):
    n = ctypes.c_size_t(0)
    assert L.csa_attend_workspace(1, 1, 32768, 128, 128, 512, 128, ctypes.byref(n)) == 0
    assert n.value == 0                                   # enough rows: no split
    assert L.hca_attend_workspace(1, 32, 1, 128, 128, 8192, 128, 128, (1 << 20) - 1,
                                  ctypes.byref(n)) == 0
    assert n.value > 0                                    # decode splits the key list
    assert L.csa_attend_workspace(1, 1, 1, 96, 128, 512, 128, ctypes.byref(n)) == EUNSUP
    assert L.csa_attend_workspace(1, 1, 1, 128, 96, 512, 128, ctypes.byref(n)) == EUNSUP
    # raw rows must cover the window of every query
    q, o, kv, r = V(128 * 128, 1), V(128 * 128, 1, out=True), V(128, 300), V(128, 128)
    st = L.csa_attend(1, 1, 1, 128, 128, 300, 4, 128, 16, 1199, 1.0, q, kv, kv, P, r, r,
                      1073, 127, o, None, 0, None)
    assert st == EINVAL and "raw rows" in err(L)
    st = L.hca_attend(1, 1, 1, 128, 128, 300, 4, 0, 1199, 1.0, q, kv, kv, r, r, 1072, 128, o,
                      None, 0, None)
    assert st == EINVAL and "window" in err(L)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(binding.CsaError):
        binding.lib()


def test_index_noalloc_rejects_before_the_device(L):
    """csa_index_topk_noalloc checks its arguments and the scratch size before
    any device call: a selection needing more than the static array (140,000
    query rows, up to 34,968 candidates: chunk lists of 2.6 GB) is refused."""
    f = L.csa_index_topk_noalloc
    q = V(256, 140000)
    assert f(1, 1, 140000, 4, 64, 35000, 4, 128, 512, 0, q, P, P, P, None) == EUNSUP
    assert "scratch" in err(L)
    assert f(1, 1, 16, 3, 64, 8192, 4, 128, 512, 0, V(192, 16), P, P, P, None) == EUNSUP   # HI
    assert f(1, 1, 16, 4, 64, 8192, 4, 128, 0, 0, q, P, P, P, None) == EINVAL     # k
    assert f(1, 1, 16, 4, 64, 8192, 4, 128, 512, 0, V(256, 16, p=0), P, P, P, None) == EINVAL
    assert "null" in err(L)
    assert f(1, 1, 1, 4, 64, 100, 4, 128, 512, 1 << 20, V(256, 1), P, P, P, None) == EINVAL
