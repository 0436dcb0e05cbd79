"""Summaries of rocprofv3 CSV output for the bench's roofline numbers.

  python -m linear_attention_token_chunked_amd.rocprof_summary stats <trace_dir> <out.txt> --cmd "<command>"
      per-kernel call count and average / min / max duration from --kernel-trace output
  python -m linear_attention_token_chunked_amd.rocprof_summary traffic <fetch_dir> <write_dir> <calib_mib> \\
        <traffic.json> <out.txt> --workload family=name [...] --cmd "<command>"
      HBM bytes per call of every measured family of kernels from a FETCH_SIZE run and a
      WRITE_SIZE run of the same command.  Each counter is scaled by the factor that makes
      it read the known size of a plain device copy in the same run (calib_mib MiB read and
      written once).  A call's bytes are those of all the family's dispatches divided by the
      number of calls (dispatches of the family's main kernel).  Records are merged into
      traffic.json under "family@workload".
  python -m linear_attention_token_chunked_amd.rocprof_summary counters <dir> <out.txt> --kernel SUBSTR \\
        --cmd "<command>"
      per-dispatch averages of every counter collected for the kernels whose name holds SUBSTR

Each traffic record holds a hash of the source files its family is built from; bench.py
reports the traffic only while those files still have that hash.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc")

# Source files of each family of kernels the bench measures.
# Every file a family's kernels are compiled from counts, the shared headers included.
SOURCES = {
    "prefill": ["prefill.hip", "seg.hip", "device_common.hpp", "launch.hpp", "plan.cpp"],
    "bwd": ["prefill.hip", "bwd.hip", "device_common.hpp", "launch.hpp", "plan.cpp"],
    "decode": ["decode.hip", "lane_sums.hpp", "device_common.hpp", "launch.hpp"],
    "verify": ["verify.hip", "lane_sums.hpp", "device_common.hpp", "launch.hpp"],
    "epilogue": ["epilogue.hip", "device_common.hpp", "launch.hpp"],
    "short_conv": ["conv.hip", "device_common.hpp", "launch.hpp"],
}
# The kernel whose dispatches count the family's calls.
MAIN = {"prefill": ("prefill", "prefill_seg"), "bwd": ("bwd_dlocal",), "decode": ("decode",), "verify": ("verify",),
        "epilogue": ("epilogue",), "short_conv": ("short_conv",)}


def sources_hash(family):
    h = hashlib.sha256()
    for f in SOURCES[family]:
        path = os.path.join(CSRC, f)
        if os.path.exists(path):
            h.update(f.encode())
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def _find(d, suffix):
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    return files


def kind(name):
    """(family, kernel) of a dispatch, or None for kernels that are not measured."""
    if "prefill_kernel" in name:  # the two last template flags: the saving variant a backward pass
        if name.endswith("Lb1ELb0EEEvNS0_6ParamsE"):  # runs, and the segmented variant of long rows
            return ("bwd", "prefill_save")
        return ("prefill", "prefill_seg" if name.endswith("Lb0ELb1EEEvNS0_6ParamsE") else "prefill")
    for sub, fam, k in (("order_kernel", "prefill", "order"), ("seg_correct_kernel", "prefill", "seg_correct"),
                        ("seg_scan_step_kernel", "prefill", "seg_scan"),
                        ("dstate_kernel", "bwd", "bwd_dstate"), ("dlocal_kernel", "bwd", "bwd_dlocal"),
                        ("chunk_prefix_kernel", "bwd", "bwd_prefix"),
                        ("decode_kernel", "decode", "decode"), ("verify_kernel", "verify", "verify"),
                        ("norm_gate_kernel", "epilogue", "epilogue"), ("conv_kernel", "short_conv", "short_conv")):
        if sub in name:
            return (fam, k)
    if "copyBuffer" in name:  # the runtime's device copy: the calibration copy and the bench's own copies
        return ("copy", "copy")
    return None


def stats(trace_dir, out, cmd):
    rows = []
    for f in _find(trace_dir, "kernel_trace.csv"):
        rows += list(csv.DictReader(open(f)))
    per = collections.defaultdict(list)
    for r in rows:
        per[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# rocprofv3 kernel trace summary", f"# command: {cmd}", "",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  kernel"]
    for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(d):6d} {sum(d) / len(d):10.2f} {min(d):10.2f} {max(d):10.2f}  {name[:150]}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter(d, counter):
    out = collections.defaultdict(list)  # (family, kernel) -> per-dispatch values (KiB)
    for f in _find(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            k = kind(r["Kernel_Name"])
            if k:
                out[k].append(float(r["Counter_Value"]))
    return out


def traffic(fetch_dir, write_dir, calib_mib, out_json, out_txt, cmd, workloads):
    calib = calib_mib * 1024 * 1024
    fetch = _counter(fetch_dir, "FETCH_SIZE")
    write = _counter(write_dir, "WRITE_SIZE")
    f_fetch = calib / (max(fetch[("copy", "copy")]) * 1024)  # the calibration copy is the largest copy
    f_write = calib / (max(write[("copy", "copy")]) * 1024)
    try:
        res = json.load(open(out_json))
    except (OSError, ValueError):
        res = {}
    res["calibration"] = {"copy_bytes": calib, "fetch_factor": f_fetch, "write_factor": f_write}
    lines = ["# HBM traffic per call from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB), scaled by the",
             f"# factor that makes a plain {calib_mib} MiB device copy read and write {calib_mib} MiB.",
             f"# command: {cmd}", f"# fetch factor {f_fetch:.4f}, write factor {f_write:.4f}", ""]
    for fam, wl in workloads.items():
        kernels = sorted(k for (f, k) in fetch if f == fam)
        calls = sum(len(fetch[(fam, k)]) for k in kernels if k in MAIN[fam])
        if not calls:
            continue
        rd = sum(sum(fetch[(fam, k)]) for k in kernels) * 1024 * f_fetch / calls
        wr = sum(sum(write.get((fam, k), [])) for k in kernels) * 1024 * f_write / calls
        res[f"{fam}@{wl}"] = {"family": fam, "workload": wl, "sources_sha256_16": sources_hash(fam),
                              "read_bytes_per_call": rd, "write_bytes_per_call": wr, "bytes_per_call": rd + wr,
                              "calls": calls}
        lines.append(f"{fam:10s} {wl:22s} read {rd / 1e6:10.2f} MB  write {wr / 1e6:10.2f} MB  "
                     f"total {(rd + wr) / 1e6:10.2f} MB per call  ({calls} calls)")
        for k in kernels:
            n = len(fetch[(fam, k)])
            kr = sum(fetch[(fam, k)]) * 1024 * f_fetch / n
            kw = sum(write.get((fam, k), [0.0])) * 1024 * f_write / max(1, len(write.get((fam, k), [])))
            lines.append(f"    {k:14s} read {kr / 1e6:10.2f} MB  write {kw / 1e6:10.2f} MB per dispatch "
                         f"({n} dispatches)")
    json.dump(res, open(out_json, "w"), indent=1, sort_keys=True)
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters(d, out, substr, cmd):
    per = collections.defaultdict(list)
    grid = set()
    for f in _find(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if substr in r["Kernel_Name"]:
                per[r["Counter_Name"]].append(float(r["Counter_Value"]))
                grid.add((r["Kernel_Name"][:120], r["Grid_Size"], r.get("Workgroup_Size", "")))
    lines = [f"# rocprofv3 counters per dispatch (average) of kernels matching '{substr}'", f"# command: {cmd}"]
    lines += [f"# kernel {k} grid {g} workgroup {w}" for k, g, w in sorted(grid)]
    lines.append("")
    for name, v in sorted(per.items()):
        lines.append(f"{name:28s} {sum(v) / len(v):18,.0f}   ({len(v)} dispatches)")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("trace_dir")
    s.add_argument("out")
    s.add_argument("--cmd", default="")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("calib_mib", type=int)
    t.add_argument("out_json")
    t.add_argument("out_txt")
    t.add_argument("--cmd", default="")
    t.add_argument("--workload", action="append", default=[], help="family=workload measured in this run")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("out")
    c.add_argument("--kernel", required=True)
    c.add_argument("--cmd", default="")
    a = ap.parse_args()
    if a.what == "stats":
        stats(a.trace_dir, a.out, a.cmd)
    elif a.what == "traffic":
        traffic(a.fetch_dir, a.write_dir, a.calib_mib, a.out_json, a.out_txt, a.cmd,
                dict(x.split("=", 1) for x in a.workload))
    else:
        counters(a.dir, a.out, a.kernel, a.cmd)


if __name__ == "__main__":
    main()
