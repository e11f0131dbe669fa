"""The rocprofv3 CSV summariser behind profiles/: step matching, copy scaling
and per-stage bytes on small synthetic counter files (CPU only)."""
import csv
import json

import pytest

from compressed_sparse_attention_04_amd import profsum as P

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, rows):
    """rows: (dispatch, kernel, counter, value); a dispatch may repeat a
    counter (several counter instances), which the summariser adds up."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for d, k, c, v in rows:
            w.writerow({"Correlation_Id": d, "Dispatch_Id": d, "Kernel_Name": k,
                        "Counter_Name": c, "Counter_Value": v})


K = {"scan": "void csa::k_dscan<unsigned short, 4>(x)", "merge": "void csa::k_dmerge<1>(y)",
     "att": "void csa::k_attend_bf16<4, 128>(z)", "cmb": "void csa::k_attend_combine<u>(w)",
     "other": "void at::native::fill_kernel(v)"}


def decode_rows(counter, scale):
    """Two csa_decode_1m steps, a stray kernel before, between and after."""
    rows, d = [], 0
    for step in range(2):
        d += 1
        rows.append((d, K["other"], counter, 1e6))
        for name, kib in (("scan", 100.0), ("merge", 2.0), ("att", 30.0), ("cmb", 5.0)):
            d += 1
            # two counter instances per dispatch
            rows.append((d, K[name], counter, kib * scale / 2))
            rows.append((d, K[name], counter, kib * scale / 2))
    d += 1
    rows.append((d, K["other"], counter, 1e6))
    return rows


def test_steps_match_the_workload_pattern(tmp_path):
    p = tmp_path / "f.csv"
    write_csv(p, decode_rows("FETCH_SIZE", 1.0))
    steps = P.steps_of(P.read_dispatches(p), "csa_decode_1m")
    assert len(steps) == 2
    assert [s for s, _ in steps[0]] == ["index_topk", "index_topk", "csa_attend", "csa_attend"]
    # an incomplete pattern is not a step
    assert P.steps_of(P.read_dispatches(p)[:4], "csa_decode_1m") == []


def test_traffic_scales_by_the_copy_and_records(tmp_path):
    # the copy reads half its bytes on FETCH_SIZE and all of them on WRITE_SIZE
    copy_kib = 262144.0
    write_csv(tmp_path / "cf.csv", [(1, K["other"], "FETCH_SIZE", copy_kib / 2),
                                    (2, K["other"], "FETCH_SIZE", 10.0)])
    write_csv(tmp_path / "cw.csv", [(1, K["other"], "WRITE_SIZE", copy_kib)])
    write_csv(tmp_path / "f.csv", decode_rows("FETCH_SIZE", 1.0))
    write_csv(tmp_path / "w.csv", decode_rows("WRITE_SIZE", 0.5))
    fs, ws, res = P.traffic("csa_decode_1m", tmp_path / "f.csv", tmp_path / "w.csv",
                            tmp_path / "cf.csv", tmp_path / "cw.csv")
    assert fs == pytest.approx(2.0) and ws == pytest.approx(1.0)
    # index_topk: scan + merge = 102 KiB counted, scaled by 2 on reads
    assert res["index_topk"]["read"] == pytest.approx(102 * 1024 * 2)
    assert res["index_topk"]["write"] == pytest.approx(51 * 1024)
    assert res["csa_attend"]["bytes"] == pytest.approx(35 * 1024 * 2 + 17.5 * 1024)
    assert res["csa_attend"]["digest"] == P.source_digest(P.STAGE_SOURCES["csa_attend"])
    rec = tmp_path / "traffic.json"
    P.record_traffic(rec, "csa_decode_1m", fs, ws, res)
    e = json.load(open(rec))["entries"]["csa_decode_1m/index_topk"]
    assert e["bytes"] == pytest.approx(res["index_topk"]["bytes"])


def test_counter_means_per_kernel(tmp_path):
    write_csv(tmp_path / "c.csv", [(1, K["att"], "SQ_WAVES", 4.0), (2, K["att"], "SQ_WAVES", 8.0),
                                   (1, K["att"], "MfmaUtil", 30.0), (3, K["other"], "SQ_WAVES", 1.0)])
    md = P.counter_means(tmp_path / "c.csv")
    row = [l for l in md.splitlines() if "k_attend_bf16" in l][0]
    assert "| 6 |" in row.replace("6.0", "6")          # mean of 4 and 8
    assert "fill_kernel" not in md                      # library kernels only


def test_digest_ignores_comments_and_spacing(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    src.mkdir()
    (src / "a.hip").write_text("int x = 1; // note\n/* block */ int y;\n")
    monkeypatch.setattr(P, "CSRC", str(src))
    d1 = P.source_digest(["a.hip"])
    (src / "a.hip").write_text("int x = 1;   int y;  // other note\n")
    assert P.source_digest(["a.hip"]) == d1
    (src / "a.hip").write_text("int x = 2; int y;\n")
    assert P.source_digest(["a.hip"]) != d1
