"""Summaries of rocprofv3 CSV output for the records kept under profiles/.

Measurement tooling: nothing in the library imports this module.  It reads
the CSV files that ``rocprofv3 --output-format csv`` writes for
``bench.py`` runs and gives

* kernel durations (``--kernel-trace --stats`` runs),
* HBM bytes per launch of each bench stage, from a ``--pmc FETCH_SIZE`` run
  and a ``--pmc WRITE_SIZE`` run of one workload, each scaled by what the
  same counter reads for a plain device copy of known size
  (``bench.py --calibrate-copy``), and recorded in profiles/traffic.json
  with a digest of the stage's kernel sources,
* per-kernel means of any other counters.

Usage (paths are the rocprofv3 output directories' CSV files):

  python -m compressed_sparse_attention_04_amd.profsum stats TRACE_STATS_CSV
  python -m compressed_sparse_attention_04_amd.profsum counters COUNTER_CSV
  python -m compressed_sparse_attention_04_amd.profsum traffic WORKLOAD FETCH_CSV WRITE_CSV \\
      CAL_FETCH_CSV CAL_WRITE_CSV [--record profiles/traffic.json]
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# Kernel sources behind each stage of bench.py: a recorded traffic figure is
# valid only while the digest of these sources still matches.
_IDX = ["indexer.hip", "index_stream.hip", "index_decode.hip", "wave_select.h", "select.h",
        "mxfp4.h", "fp4_tiles.h", "common.h", "internal.h"]
STAGE_SOURCES = {
    "index_topk": _IDX,
    "csa_attend": ["attend.hip", "common.h", "internal.h"],
    "hca_attend": ["attend.hip", "common.h", "internal.h"],
    "csa_attend_fp8": ["attend_fp8.hip", "attend_common.h", "attend.hip", "common.h",
                       "internal.h"],
    "hca_attend_fp8": ["attend_fp8.hip", "attend_common.h", "attend.hip", "common.h",
                       "internal.h"],
    "compress_m4": ["compress.hip", "common.h", "internal.h"],
    "compress_m128": ["compress.hip", "common.h", "internal.h"],
    "quantize_keys": ["mxfp4.hip", "mxfp4.h", "common.h", "internal.h"],
}

# The library kernels one step of each bench workload launches, in order:
# (stage, kernel name fragment).
STEP_KERNELS = {
    "pair_prefill_128k": [("compress_m4", "k_compress_small"), ("compress_m4", "k_compress_small"),
                          ("quantize_keys", "k_quant_mxfp4"), ("index_topk", "k_index_stream"),
                          ("csa_attend", "k_attend_bf16"),
                          ("compress_m128", "k_compress_large"),
                          ("compress_m128", "k_compress_large"),
                          ("hca_attend", "k_attend_bf16")],
    "csa_prefill_32k": [("compress_m4", "k_compress_small"), ("compress_m4", "k_compress_small"),
                        ("quantize_keys", "k_quant_mxfp4"), ("index_topk", "k_index_stream"),
                        ("csa_attend", "k_attend_bf16")],
    "hca_decode_1m": [("hca_attend", "k_attend_bf16"), ("hca_attend", "k_attend_combine")],
    "csa_decode_1m": [("index_topk", "k_dscan"), ("index_topk", "k_dmerge"),
                      ("csa_attend", "k_attend_bf16"), ("csa_attend", "k_attend_combine")],
    "hca_decode_1m_fp8": [("hca_attend_fp8", "k_attend_fp8"),
                          ("hca_attend_fp8", "k_attend_combine")],
    "csa_decode_1m_fp8": [("index_topk", "k_dscan"), ("index_topk", "k_dmerge"),
                          ("csa_attend_fp8", "k_attend_fp8"),
                          ("csa_attend_fp8", "k_attend_combine")],
}


def source_digest(files):
    """sha1 over the kernel sources with comments and blank space removed."""
    h = hashlib.sha1()
    for f in files:
        text = open(os.path.join(CSRC, f)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(f.encode())
        h.update(re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()


def short_name(kernel):
    """'void csa::k_attend_bf16<4, 128, ...>(...)' -> 'csa::k_attend_bf16<4, 128, ...>'"""
    name = kernel.split("(")[0]
    return name[5:] if name.startswith("void ") else name


def read_dispatches(path):
    """Counter CSV -> [(dispatch id, kernel, {counter: value})] in dispatch order."""
    per = collections.OrderedDict()
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            e = per.setdefault(d, (r["Kernel_Name"], {}))
            e[1][r["Counter_Name"]] = e[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [(d, k, c) for d, (k, c) in sorted(per.items())]


def steps_of(dispatches, workload):
    """The complete steps of a workload found in a dispatch list: runs of
    consecutive library dispatches that match its kernel pattern."""
    pat = STEP_KERNELS[workload]
    lib = [x for x in dispatches if "csa::" in x[1]]
    out, i = [], 0
    while i + len(pat) <= len(lib):
        if all(frag in lib[i + j][1] for j, (_, frag) in enumerate(pat)):
            out.append([(pat[j][0], lib[i + j]) for j in range(len(pat))])
            i += len(pat)
        else:
            i += 1
    return out


def copy_scale(path, counter, nbytes):
    """Scale of a byte counter: bytes a plain copy moves over what the counter
    reads for it (the dispatch with the largest reading)."""
    vals = [c.get(counter, 0.0) for _, _, c in read_dispatches(path)]
    return nbytes / (max(vals) * 1024.0)


def traffic(workload, fetch_csv, write_csv, cal_fetch, cal_write, copy_bytes=256 << 20):
    """Scaled HBM bytes (read, write) per launch of each stage, averaged over
    the complete steps of both runs."""
    fs = copy_scale(cal_fetch, "FETCH_SIZE", copy_bytes)
    ws = copy_scale(cal_write, "WRITE_SIZE", copy_bytes)
    res = {}
    for path, counter, scale, key in ((fetch_csv, "FETCH_SIZE", fs, "read"),
                                      (write_csv, "WRITE_SIZE", ws, "write")):
        steps = steps_of(read_dispatches(path), workload)
        if not steps:
            raise SystemExit(f"no complete {workload} step in {path}")
        acc = collections.defaultdict(float)
        for st in steps:
            for stage, (_, _, c) in st:
                acc[stage] += c.get(counter, 0.0) * 1024.0 * scale
        for stage, v in acc.items():
            res.setdefault(stage, {})[key] = v / len(steps)
    for stage, e in res.items():
        e["bytes"] = e["read"] + e["write"]
        e["digest"] = source_digest(STAGE_SOURCES[stage])
    return fs, ws, res


def record_traffic(path, workload, fs, ws, res):
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        rec = {"entries": {}}
    rec["fetch_scale"], rec["write_scale"] = fs, ws
    for stage, e in res.items():
        rec["entries"][f"{workload}/{stage}"] = e
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")


def kernel_stats(path):
    """rocprofv3 kernel_stats CSV -> markdown rows (name, calls, avg, min, max us)."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if "csa::" not in r["Name"]:
                continue
            rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                         float(r["TotalDurationNs"]) / 1e3))
    rows.sort(key=lambda x: -x[5])
    lines = ["| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
    lines += [f"| `{n}` | {c} | {a:.2f} | {lo:.2f} | {hi:.2f} |" for n, c, a, lo, hi, _ in rows]
    return "\n".join(lines)


def counter_means(path):
    """Counter CSV -> markdown rows of per-kernel mean values."""
    acc = collections.OrderedDict()
    for _, k, c in read_dispatches(path):
        if "csa::" not in k:
            continue
        e = acc.setdefault(short_name(k), collections.defaultdict(list))
        for n, v in c.items():
            e[n].append(v)
    names = sorted({n for e in acc.values() for n in e})
    lines = ["| kernel | dispatches | " + " | ".join(names) + " |",
             "|---|---|" + "---|" * len(names)]
    for k, e in acc.items():
        nd = max(len(v) for v in e.values())
        vals = [f"{sum(e[n]) / len(e[n]):.4g}" if e.get(n) else "" for n in names]
        lines.append(f"| `{k}` | {nd} | " + " | ".join(vals) + " |")
    return "\n".join(lines)


def main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        print(kernel_stats(argv[1]))
    elif len(argv) >= 2 and argv[0] == "counters":
        print(counter_means(argv[1]))
    elif len(argv) >= 6 and argv[0] == "traffic":
        fs, ws, res = traffic(*argv[1:6])
        if "--record" in argv:
            record_traffic(argv[argv.index("--record") + 1], argv[1], fs, ws, res)
        print(f"FETCH_SIZE scale {fs:.4f}, WRITE_SIZE scale {ws:.4f}")
        print("| stage | read GB | write GB | total GB |\n|---|---|---|---|")
        for stage, e in res.items():
            print(f"| {stage} | {e['read'] / 1e9:.4f} | {e['write'] / 1e9:.4f} | "
                  f"{e['bytes'] / 1e9:.4f} |")
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
