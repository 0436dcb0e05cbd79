"""Summaries of rocprofv3 CSV output for the bench's roofline numbers.

  python -m linear_attention_token_chunked_amd.rocprof_summary stats <trace_dir> <out.txt> --cmd "<command>"
      per-kernel call count and average / min / max duration from --kernel-trace output
  python -m linear_attention_token_chunked_amd.rocprof_summary traffic <fetch_dir> <write_dir> <calib_mib> \
        <out.json> <out.txt> --cmd "<command>"
      HBM bytes per launch of the measured kernels from a FETCH_SIZE run and a
      WRITE_SIZE run.  Each counter is scaled by the factor that makes it read the known
      size of a plain device copy in the same run (calib_mib MiB read and written once).

The traffic JSON records a hash of each kernel's source file; bench.py reports the
traffic only while the source still has that hash.
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
SOURCES = {
    "prefill": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "prefill.hip"),
    "decode": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "decode.hip"),
    "prefill_save": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "prefill.hip"),
    "bwd_dstate": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "bwd.hip"),
    "bwd_dlocal": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "bwd.hip"),
    "verify": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "verify.hip"),
    "epilogue": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "epilogue.hip"),
    "short_conv": os.path.join(ROOT, "linear_attention_token_chunked_amd", "csrc", "conv.hip"),
}


def _find(d, suffix):
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    return files


def _kind(name):
    if "prefill_kernel" in name:  # the last two template flags: the saving variant a backward pass
        if name.endswith("Lb1ELb0EEEvNS0_6ParamsE"):  # runs, and the segmented variant of long rows
            return "prefill_save"
        return "prefill_seg" if name.endswith("Lb0ELb1EEEvNS0_6ParamsE") else "prefill"
    if "seg_correct_kernel" in name:
        return "seg_correct"
    if "seg_scan_step_kernel" in name:
        return "seg_scan"
    if "dstate_kernel" in name:
        return "bwd_dstate"
    if "dlocal_kernel" in name:
        return "bwd_dlocal"
    if "decode_kernel" in name:
        return "decode"
    if "verify_kernel" in name:
        return "verify"
    if "norm_gate_kernel" in name:
        return "epilogue"
    if "conv_kernel" in name:
        return "short_conv"
    if "copyBuffer" in name or "copy" in name.lower():
        return "copy"
    return None


def stats(trace_dir, out, cmd):
    rows = []
    for f in _find(trace_dir, "kernel_trace.csv"):
        rows += list(csv.DictReader(open(f)))
    per = collections.defaultdict(list)
    for r in rows:
        per[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# rocprofv3 kernel trace summary", f"# command: {cmd}", "",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10}  kernel"]
    for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(d):6d} {sum(d) / len(d):10.2f} {min(d):10.2f} {max(d):10.2f}  {name[:150]}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_per_dispatch(d, counter):
    out = collections.defaultdict(list)
    for f in _find(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            k = _kind(r["Kernel_Name"])
            if k:
                out[k].append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def traffic(fetch_dir, write_dir, calib_mib, out_json, out_txt, cmd, workloads):
    calib = calib_mib * 1024 * 1024
    fetch = _counter_per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _counter_per_dispatch(write_dir, "WRITE_SIZE")
    big = lambda lst: max(v for _, _, v in lst)  # the calibration copy is the largest copy dispatch
    f_fetch = calib / (big(fetch["copy"]) * 1024)
    f_write = calib / (big(write["copy"]) * 1024)
    res = {"calibration": {"copy_bytes": calib, "fetch_factor": f_fetch, "write_factor": f_write}}
    lines = ["# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB), scaled by the",
             f"# factor that makes a plain {calib_mib} MiB device copy read and write {calib_mib} MiB.",
             f"# command: {cmd}", f"# fetch factor {f_fetch:.4f}, write factor {f_write:.4f}", ""]
    for k in ("prefill", "decode", "prefill_save", "bwd_dstate", "bwd_dlocal", "verify", "epilogue", "short_conv"):
        if k not in fetch or k not in write:
            continue
        fr = sum(v for _, _, v in fetch[k]) / len(fetch[k]) * 1024 * f_fetch
        wr = sum(v for _, _, v in write[k]) / len(write[k]) * 1024 * f_write
        res[k] = {"workload": workloads[k], "source_sha256_16": hashlib.sha256(open(SOURCES[k], "rb").read())
                  .hexdigest()[:16], "read_bytes_per_launch": fr, "write_bytes_per_launch": wr,
                  "bytes_per_launch": fr + wr, "dispatches": len(fetch[k])}
        lines.append(f"{k:12s} {workloads[k]:22s} read {fr / 1e6:10.2f} MB  write {wr / 1e6:10.2f} MB  "
                     f"total {(fr + wr) / 1e6:10.2f} MB per launch  ({len(fetch[k])} dispatches)")
    json.dump(res, open(out_json, "w"), indent=1)
    open(out_txt, "w").write("\n".join(lines) + "\n")
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
    t.add_argument("--prefill-workload", default="prefill_b4_t4096")
    t.add_argument("--decode-workload", default="decode_n256")
    t.add_argument("--verify-workload", default="verify_n256_t4")
    t.add_argument("--epilogue-workload", default="epilogue_b4_t4096")
    t.add_argument("--short-conv-workload", default="short_conv_q_b4_t4096")
    a = ap.parse_args()
    if a.what == "stats":
        stats(a.trace_dir, a.out, a.cmd)
    else:
        traffic(a.fetch_dir, a.write_dir, a.calib_mib, a.out_json, a.out_txt, a.cmd,
                {"prefill": a.prefill_workload, "decode": a.decode_workload, "prefill_save": a.prefill_workload,
                 "bwd_dstate": a.prefill_workload, "bwd_dlocal": a.prefill_workload,
                 "verify": a.verify_workload, "epilogue": a.epilogue_workload,
                 "short_conv": a.short_conv_workload})


if __name__ == "__main__":
    main()
