"""Summaries of rocprofv3 output for the profiles/ folder.

  python -m structured_sparse_matrix_amd.profiling kernels TRACE_CSV [--match snm] [--skip N]
         [--groups G] [--alone] [--dispatch A:B]
      Markdown table of kernel dispatch durations (calls, mean, median, min, max) from a
      `rocprofv3 --kernel-trace -f csv` run. --groups G splits each kernel's dispatches, in
      dispatch order, into G equal consecutive groups reported as separate rows (a program
      that times the same kernel on G inputs one after the other). --alone keeps only the
      dispatches that overlapped no other dispatch (a program that also runs kernels
      concurrently on several streams).

  python -m structured_sparse_matrix_amd.profiling traffic --fetch FETCH_CSV --write WRITE_CSV
         --match NAME --calibration-bytes N [--sources decode|wide] [--groups G --labels L,..]
         [--workload W] [--command CMD]
      HBM traffic per launch of the kernels whose name contains NAME, from two
      `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of the same program. Each
      counter is scaled by what it reads for the largest plain copy kernel (N bytes read
      and N bytes written) dispatched before the first matching kernel. Prints JSON with
      the kernel-source hash that bench.py compares against.

  python -m structured_sparse_matrix_amd.profiling mfma COUNTER_CSV --match NAME [--groups G]
         [--cus 256] [--command CMD]
      Matrix-core use of the kernels whose name contains NAME, from one `rocprofv3 --pmc
      SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_BUSY_CU_CYCLES`
      run: per dispatch (split in order into G groups) the busy fraction of the matrix cores
      (MFMA busy cycles, summed over SIMDs, over the per-XCD GUI-active cycles x CUs x 4
      SIMDs; GRBM_GUI_ACTIVE is summed over the XCDs) and the fp16 matrix operations
      (MOPS x 512). Prints JSON with the wide-kernel source hash.

  python -m structured_sparse_matrix_amd.profiling counters COUNTER_CSV --match NAME
         [--sources attention|wide|decode] [--workload W] [--command CMD]
      Per-dispatch means of every counter of one `rocprofv3 --pmc ...` run for the kernels
      whose name contains NAME (summed over the per-XCD / per-instance rows of a dispatch),
      with the derived per-wave figures where the counters are present: instructions per
      wave (SQ_INSTS_* / SQ_WAVES) and the share of wave cycles spent issuing VALU
      instructions (SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES) or waiting (SQ_WAIT_INST_ANY /
      SQ_WAVE_CYCLES). Prints JSON with the source hash of the named kernel family.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
DECODE_KERNEL_SOURCES = ("spmm_skinny.hip", "device_common.hpp", "lds_dma.hpp")
WIDE_KERNEL_SOURCES = ("spmm_wide.hip", "spmm_vnm_big.hip", "lds_dma.hpp", "wide_layout.hpp", "elem.hpp",
                       "device_common.hpp")
ATTENTION_KERNEL_SOURCES = ("attention.hip", "elem.hpp", "device_common.hpp")
SOURCES = {"decode": DECODE_KERNEL_SOURCES, "wide": WIDE_KERNEL_SOURCES, "attention": ATTENTION_KERNEL_SOURCES}


def kernel_source_hash(files=DECODE_KERNEL_SOURCES) -> str:
    """Hash of the kernel sources a counter summary was taken on."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _alone(spans):
    """Flags, per (start, end) span in dispatch order, whether no other span overlaps it."""
    order = sorted(range(len(spans)), key=lambda i: spans[i][0])
    flags = [True] * len(spans)
    reach = None   # latest end among the spans that start earlier
    for pos, i in enumerate(order):
        b, e = spans[i]
        if reach is not None and reach > b:
            flags[i] = False
        if pos + 1 < len(order) and spans[order[pos + 1]][0] < e:
            flags[i] = False
        reach = e if reach is None else max(reach, e)
    return flags


def _durations(path, match, skip, alone=False, dispatch=None):
    rows = list(csv.DictReader(open(path)))
    spans = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    keep = _alone(spans) if alone else [True] * len(rows)
    by = {}
    for r, (b, e), k in zip(rows, spans, keep):
        name = r["Kernel_Name"]
        if not k or (match and match not in name):
            continue
        if dispatch and not dispatch[0] <= int(r["Dispatch_Id"]) <= dispatch[1]:
            continue
        by.setdefault(name, []).append(e - b)
    return {k: v[skip:] if len(v) > skip else v for k, v in by.items()}


def kernels_table(path, match, skip, groups=1, alone=False, dispatch=None):
    rows = ["| kernel | calls | mean us | median us | min us | max us |", "|---|---|---|---|---|---|"]
    for name, ds in sorted(_durations(path, match, skip, alone, dispatch).items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) < 110 else name[:107] + "..."
        n = len(ds) // groups if groups > 1 and len(ds) % groups == 0 else len(ds)
        parts = [ds[i:i + n] for i in range(0, len(ds), n)]
        for g, part in enumerate(parts):
            label = f"`{short}`" + (f" ({g + 1} of {len(parts)})" if len(parts) > 1 else "")
            rows.append(f"| {label} | {len(part)} | {statistics.mean(part) / 1e3:.2f} | "
                        f"{statistics.median(part) / 1e3:.2f} | {min(part) / 1e3:.2f} | {max(part) / 1e3:.2f} |")
    return "\n".join(rows)


def _counter_rows(path, counter):
    out = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0))
    out.sort()
    return out


def traffic(fetch_csv, write_csv, match, calibration_bytes, groups=1):
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
    write = _counter_rows(write_csv, "WRITE_SIZE")
    first = next(i for i, (_, n, _) in enumerate(fetch) if match in n)
    calib_f = max((b, n) for _, n, b in fetch[:first] if "snm" not in n)
    firstw = next(i for i, (_, n, _) in enumerate(write) if match in n)
    calib_w = max((b, n) for _, n, b in write[:firstw] if "snm" not in n)
    ff = calib_f[0] / calibration_bytes
    fw = calib_w[0] / calibration_bytes
    kf = [b / ff for _, n, b in fetch if match in n]
    kw = [b / fw for _, n, b in write if match in n]
    n = min(len(kf), len(kw))
    per = [kf[i] + kw[i] for i in range(n)]
    out = {
        "kernel_match": match,
        "launches": n,
        "fetch_bytes_per_launch_avg": statistics.mean(kf[:n]),
        "write_bytes_per_launch_avg": statistics.mean(kw[:n]),
        "bytes_per_launch_avg": statistics.mean(per),
        "calibration": {"bytes": calibration_bytes, "fetch_factor": ff, "write_factor": fw,
                        "fetch_kernel": calib_f[1][:80], "write_kernel": calib_w[1][:80]},
    }
    if groups > 1 and n % groups == 0:
        g = n // groups
        out["groups"] = [{"launches": g,
                          "fetch_bytes_per_launch_avg": statistics.mean(kf[i:i + g]),
                          "write_bytes_per_launch_avg": statistics.mean(kw[i:i + g]),
                          "bytes_per_launch_avg": statistics.mean(per[i:i + g])}
                         for i in range(0, n, g)]
    return out


def mfma(csv_path, match, groups=1, cus=256, xcds=8):
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if match not in r["Kernel_Name"]:
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(per)
    n = len(ids) // groups if groups > 1 and len(ids) % groups == 0 else len(ids)
    out = []
    for g in range(0, len(ids), n):
        rows = [per[i] for i in ids[g:g + n]]
        busy = statistics.mean(r["SQ_VALU_MFMA_BUSY_CYCLES"] for r in rows)
        gui = statistics.mean(r["GRBM_GUI_ACTIVE"] for r in rows)
        mops = statistics.mean(r["SQ_INSTS_VALU_MFMA_MOPS_F16"] for r in rows)
        out.append({"dispatches": len(rows), "mfma_busy_cycles": busy,
                    "gui_active_cycles_per_xcd": gui / xcds,
                    "mfma_busy_frac": busy / (gui / xcds * cus * 4),
                    "fp16_matrix_ops": mops * 512.0,
                    "busy_cu_cycles": statistics.mean(r["SQ_BUSY_CU_CYCLES"] for r in rows)})
    return {"kernel_match": match, "groups": out, "cus": cus, "xcds": xcds}


def counters(csv_path, match):
    per = {}
    name = None
    for r in csv.DictReader(open(csv_path)):
        if match not in r["Kernel_Name"]:
            continue
        name = name or r["Kernel_Name"]
        d = per.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    rows = [per[i] for i in sorted(per)]
    keys = sorted({k for r in rows for k in r})
    mean = {k: statistics.mean(r[k] for r in rows if k in r) for k in keys}
    out = {"kernel_match": match, "kernel_name": (name or "")[:120], "dispatches": len(rows), "per_dispatch_mean": mean}
    derived = {}
    waves = mean.get("SQ_WAVES")
    if waves:
        for k in keys:
            if k.startswith("SQ_INSTS_"):
                derived[k + "_per_wave"] = mean[k] / waves
    cyc = mean.get("SQ_WAVE_CYCLES")
    if cyc:
        for k in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY"):
            if k in mean:
                derived[k + "_share_of_wave_cycles"] = mean[k] / cyc
    out["derived"] = derived
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("trace")
    k.add_argument("--match", default="")
    k.add_argument("--skip", type=int, default=0)
    k.add_argument("--groups", type=int, default=1)
    k.add_argument("--alone", action="store_true",
                   help="only dispatches that overlapped no other dispatch in time")
    k.add_argument("--dispatch", default="", help="A:B -- only dispatch ids A..B (inclusive)")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--match", required=True)
    t.add_argument("--calibration-bytes", type=int, required=True)
    t.add_argument("--command", default="")
    t.add_argument("--sources", choices=("decode", "wide"), default="decode",
                   help="kernel sources whose hash is recorded: the decode or the wide products")
    t.add_argument("--workload", default="")
    t.add_argument("--groups", type=int, default=1,
                   help="split the matching dispatches, in order, into G equal groups")
    t.add_argument("--labels", default="", help="comma-separated names of the groups")
    m = sub.add_parser("mfma")
    m.add_argument("counters")
    m.add_argument("--match", required=True)
    m.add_argument("--groups", type=int, default=1)
    m.add_argument("--cus", type=int, default=256)
    m.add_argument("--xcds", type=int, default=8)
    m.add_argument("--labels", default="", help="comma-separated names of the groups")
    m.add_argument("--workload", default="")
    m.add_argument("--command", default="")
    c = sub.add_parser("counters")
    c.add_argument("counters")
    c.add_argument("--match", required=True)
    c.add_argument("--sources", choices=tuple(SOURCES), default="attention")
    c.add_argument("--workload", default="")
    c.add_argument("--command", default="")
    a = ap.parse_args(argv)
    if a.cmd == "kernels":
        rng = tuple(int(x) for x in a.dispatch.split(":")) if a.dispatch else None
        print(kernels_table(a.trace, a.match, a.skip, a.groups, a.alone, rng))
    elif a.cmd == "counters":
        out = counters(a.counters, a.match)
        out["workload"] = a.workload
        out["kernel_source_hash"] = kernel_source_hash(SOURCES[a.sources])
        out["command"] = a.command
        print(json.dumps(out, indent=1))
    elif a.cmd == "mfma":
        out = mfma(a.counters, a.match, a.groups, a.cus, a.xcds)
        for g, lab in zip(out["groups"], [x for x in a.labels.split(",") if x]):
            g["label"] = lab
        out["workload"] = a.workload
        out["kernel_source_hash"] = kernel_source_hash(WIDE_KERNEL_SOURCES)
        out["command"] = a.command
        print(json.dumps(out, indent=1))
    else:
        out = traffic(a.fetch, a.write, a.match, a.calibration_bytes, a.groups)
        for g, lab in zip(out.get("groups", []), [x for x in a.labels.split(",") if x]):
            g["label"] = lab
        if a.workload:
            out["workload"] = a.workload
        out["kernel_source_hash"] = kernel_source_hash(
            WIDE_KERNEL_SOURCES if a.sources == "wide" else DECODE_KERNEL_SOURCES)
        out["command"] = a.command
        print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
