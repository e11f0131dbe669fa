"""The exact top-k search's range arithmetic, run on the host: compiled from
the kernels' own header (wave_select.h), it follows the widest sub-range of
every level-1 bin pass by pass and checks that every row reaches a single
key value within the static pass bound, so the pass loops of the indexer
kernels always end in the collection pass."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_sparse_attention_04_amd", "csrc")


def test_narrowing_ends_within_the_pass_bound(tmp_path):
    exe = str(tmp_path / "narrowing")
    src = os.path.join(ROOT, "tests", "native", "narrowing.cpp")
    r = subprocess.run(["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "-O2",
                        "-std=c++17", "-I", CSRC, src, "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "worst narrowing passes 4 bound 4 exact passes 6" in r.stdout
