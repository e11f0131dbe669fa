"""bench.py's command-line contract on a host without a GPU: more than one
GPU is refused with a message before anything touches a device, and the
workload and storage options parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_options_parse():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--workload", "--kv-format", "--shared-kv", "--pipeline", "--layers",
                "stack_decode_1m", "pair_prefill_128k", "hca_decode_1m", "csa_decode_1m", "all"):
        assert opt in r.stdout


def test_unknown_workload_is_rejected():
    r = run("--workload", "no_such_workload")
    assert r.returncode != 0


def test_stratified_rows_cover_the_special_positions():
    """The oracle's prefill sample: first and last 8 rows, the saturation
    point (n_cand reaches k = 512 at t = 2172 for m = 4, W = 128), window
    and block boundaries, 128 distinct rows in range."""
    sys.path.insert(0, ROOT)
    import bench
    from compressed_sparse_attention_04_amd import inputs as I
    w = I.PAIR_CSA_128K
    r = bench.stratified_rows(w)
    assert len(r) == 128 and len(set(r.tolist())) == 128
    assert r.min() >= 0 and r.max() < w.Tq
    s = set(r.tolist())
    assert set(range(8)) <= s and set(range(w.Tq - 8, w.Tq)) <= s
    assert 2171 in s and 2172 in s                      # last row below 512 candidates, first at 512
    assert {126, 127, 128, 129} <= s and {3, 4, 7, 8} <= s
    h = bench.stratified_rows(I.PAIR_HCA_128K)
    assert 128 in set(h.tolist()) and 255 in set(h.tolist())   # first candidate; block end
