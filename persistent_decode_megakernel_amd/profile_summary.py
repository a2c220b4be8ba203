"""Summaries of rocprofv3 output for the profiles/ directory.

    python -m persistent_decode_megakernel_amd.profile_summary KT_DIR FETCH_DIR WRITE_DIR OUT_STEM \
        --kernel amk_megakernel_w0_h128_q1 --calib-mib 1024 --cmd "..."

KT_DIR holds the --kernel-trace --stats CSVs; FETCH_DIR / WRITE_DIR the --pmc FETCH_SIZE /
WRITE_SIZE counter CSVs of runs that began with a plain device copy of --calib-mib MiB (the
scale of each counter is the copy's known byte count over what the counter reported for it).
Writes OUT_STEM.md (human summary) and OUT_STEM.json (per-launch HBM traffic plus a hash of the
kernel sources; the bench reports the traffic only while that hash still matches)."""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["csrc/kernels/device.h", "csrc/kernels/megakernel.hip", "csrc/sched/layout.h",
                  "csrc/sched/builder.cpp", "csrc/sched/sched_api.cpp"]


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def counters(d: str):
    """Counter values per kernel name, in dispatch order."""
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    by = {}
    for r in rows:
        by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return by


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("kt_dir")
    ap.add_argument("fetch_dir")
    ap.add_argument("write_dir")
    ap.add_argument("out_stem")
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--calib-mib", type=int, required=True)
    ap.add_argument("--calib-kernel", default="__amd_rocclr_copyBuffer")
    ap.add_argument("--cmd", default="")
    args = ap.parse_args()

    stats = list(csv.DictReader(open(_one(os.path.join(args.kt_dir, "**", "*kernel_stats.csv")))))
    f, w = counters(args.fetch_dir), counters(args.write_dir)
    calib = args.calib_mib * 1024.0  # KiB
    # the calibration copy is the first dispatch of its kernel (it runs before anything else)
    f_cal = f[args.calib_kernel][0]
    w_cal = w[args.calib_kernel][0]
    f_scale, w_scale = calib / f_cal, calib / w_cal
    fk = statistics.mean(f[args.kernel]) * f_scale
    wk = statistics.mean(w[args.kernel]) * w_scale
    traffic = (fk + wk) * 1024.0
    out = {
        "kernel": args.kernel,
        "fetch_bytes_per_launch": fk * 1024.0,
        "write_bytes_per_launch": wk * 1024.0,
        "traffic_bytes_per_launch": traffic,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "calibration": f"{args.calib_kernel}, {args.calib_mib} MiB read + written",
        "source_hash": source_hash(),
    }
    with open(args.out_stem + ".json", "w") as fo:
        json.dump(out, fo, indent=1)
    lines = [f"# rocprofv3 summary: {args.kernel}", "", "Command(s):", "", "```", args.cmd, "```", "",
             "## Kernel trace (--kernel-trace --stats)", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in stats[:12]:
        lines.append(f"| {r['Name'][:60]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    lines += ["", "## HBM counters (--pmc, one pass each)", "",
              f"- calibration: {out['calibration']}: FETCH_SIZE read {f_cal:.0f} KiB "
              f"(scale {f_scale:.4f}), WRITE_SIZE read {w_cal:.0f} KiB (scale {w_scale:.4f})",
              f"- {args.kernel}: FETCH_SIZE {statistics.mean(f[args.kernel]):.0f} KiB/launch raw, "
              f"{fk * 1024 / 1e9:.3f} GB scaled; WRITE_SIZE {statistics.mean(w[args.kernel]):.0f} "
              f"KiB/launch raw, {wk * 1024 / 1e9:.4f} GB scaled",
              f"- traffic per launch: {traffic / 1e9:.3f} GB",
              f"- kernel source hash: {out['source_hash']}"]
    with open(args.out_stem + ".md", "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print(json.dumps(out))


def lds_main(argv):
    """LDS counters of one --pmc pass (SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE and others) summed
    over the kernel's dispatches:

        python -m persistent_decode_megakernel_amd.profile_summary lds PMC_DIR OUT_STEM \
            --kernel amk_megakernel_w0_h128_q1 --cmd "..."

    The bank-conflict share is SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles the LDS spent
    resolving conflicts per cycle it was active)."""
    ap = argparse.ArgumentParser(prog="profile_summary lds")
    ap.add_argument("pmc_dir")
    ap.add_argument("out_stem")
    ap.add_argument("--kernel", required=True)
    ap.add_argument("--cmd", default="")
    args = ap.parse_args(argv)
    rows = list(csv.DictReader(open(_one(os.path.join(args.pmc_dir, "**", "*counter_collection.csv")))))
    tot, disp = {}, set()
    for r in rows:
        if r["Kernel_Name"] != args.kernel:
            continue
        disp.add(r["Dispatch_Id"])
        tot[r["Counter_Name"]] = tot.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    n = max(1, len(disp))
    per = {k: v / n for k, v in sorted(tot.items())}
    share = per.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(1.0, per.get("SQ_LDS_IDX_ACTIVE", 0.0))
    out = {"kernel": args.kernel, "dispatches": n, "per_dispatch": per,
           "bank_conflict_share": share, "source_hash": source_hash()}
    with open(args.out_stem + ".json", "w") as fo:
        json.dump(out, fo, indent=1)
    lines = [f"# rocprofv3 LDS counters: {args.kernel}", "", "Command(s):", "", "```", args.cmd, "```",
             "", f"Per dispatch, mean over {n} dispatches of {args.kernel}:", "",
             "| counter | value |", "|---|---|"]
    lines += [f"| {k} | {v:.4g} |" for k, v in per.items()]
    lines += ["", f"- bank-conflict share (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE): {share:.4f}",
              f"- kernel source hash: {out['source_hash']}"]
    with open(args.out_stem + ".md", "w") as fo:
        fo.write("\n".join(lines) + "\n")
    print(json.dumps(out))


if __name__ == "__main__":
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "lds":
        lds_main(sys.argv[2:])
    else:
        main()
