"""Turn rocprofv3 CSV output into the short summaries kept under profiles/.

    python -m matrix_core_scheduling_amd.profiling stats DIR [--kernel SUBSTR]
    python -m matrix_core_scheduling_amd.profiling counters DIR [DIR ...] [--kernel SUBSTR]
    python -m matrix_core_scheduling_amd.profiling traffic --fetch DIR --write DIR
           --copy-fetch DIR --copy-write DIR --copy-mib N --workload NAME
           [--schedule pipelined|interleaved] [--update FILE]

DIR is a rocprofv3 output directory written with --output-format csv.
Counter rows come one per hardware instance; they are summed per dispatch
and then averaged over the dispatches of the kernel.

Derived figures (MI355X: 8 XCDs, 1024 SIMDs):
  clock_GHz     = GRBM_GUI_ACTIVE / n_xcc / duration    (GRBM counts per XCD)
  mfma_busy     = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / n_xcc * simds)
  lds_conflict  = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
  HBM bytes     = counter KiB * 1024 * (known copy bytes / counter KiB of the copy)
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# Source files that determine each timed kernel's code.
KERNEL_SOURCES = {
    "pipelined": ("gemm_pipelined.hip", "device.h", "internal.h"),
    "interleaved": ("gemm_interleaved.hip", "device.h", "internal.h"),
    "tile128": ("gemm_tile128.hip", "device.h", "internal.h"),
    "attention": ("attention_fwd.hip", "device.h", "internal.h"),
    "attention4": ("attention_fwd.hip", "device.h", "internal.h"),
}
# kernel-name filter of each schedule's counter rows
KERNEL_NAMES = {"attention": "attention_fwd_kernel", "attention4": "attention_fwd4_kernel"}


def _one(d: str, pattern: str) -> str:
    hits = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return hits[0]


def agent(d: str) -> dict:
    for r in csv.DictReader(open(_one(d, "*agent_info.csv"))):
        if r.get("Name", "").startswith("gfx"):
            return r
    return {}


def kernel_stats(d: str, kernel: str = "") -> list[dict]:
    out = []
    for r in csv.DictReader(open(_one(d, "*kernel_stats.csv"))):
        if kernel in r["Name"]:
            out.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                        "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])})
    return out


def counters(dirs, kernel: str = "") -> dict:
    """{kernel name: {counter: mean per dispatch, '_duration_ns': mean, '_dispatches': n}}"""
    per = collections.defaultdict(float)
    dur = {}
    name = {}
    for d in dirs:
        for r in csv.DictReader(open(_one(d, "*counter_collection.csv"))):
            if kernel not in r["Kernel_Name"]:
                continue
            key = (d, int(r["Dispatch_Id"]))
            per[(key, r["Counter_Name"])] += float(r["Counter_Value"])
            dur[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            name[key] = r["Kernel_Name"]
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for (key, c), v in per.items():
        acc[name[key]][c].append(v)
    durs = collections.defaultdict(list)
    for key, ns in dur.items():
        durs[name[key]].append(ns)
    res = {}
    for k, cs in acc.items():
        res[k] = {c: sum(v) / len(v) for c, v in cs.items()}
        res[k]["_duration_ns"] = sum(durs[k]) / len(durs[k])
        res[k]["_dispatches"] = len(durs[k])
    return res


def derived(c: dict, n_xcc: int, simds: int) -> dict:
    out = {}
    ns = c.get("_duration_ns")
    if "GRBM_GUI_ACTIVE" in c and ns:
        cyc = c["GRBM_GUI_ACTIVE"] / n_xcc
        out["clock_GHz"] = cyc / ns
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            out["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * simds)
    if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_LDS_IDX_ACTIVE"):
        out["lds_conflict_ratio"] = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
    if "SQ_INSTS_VALU_MFMA_MOPS_F16" in c:
        out["mfma_flop"] = c["SQ_INSTS_VALU_MFMA_MOPS_F16"] * 512
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in c:
        out["mfma_flop_bf16"] = c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    if "SQ_INSTS_VALU_MFMA_MOPS_F8" in c:
        out["mfma_flop_f8"] = c["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512
    return out


def code_text(src: str) -> str:
    """C++ source with comments removed and every run of whitespace made one
    space: what the compiler sees, so editing a comment keeps the hash."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_code_hash(schedule: str = "pipelined") -> str:
    """SHA-256 of the comment-free code of the sources a timed kernel is built from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[schedule]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def traffic_key(workload: str, schedule: str = "pipelined") -> str:
    return workload if schedule == "pipelined" else f"{workload}@{schedule}"


def traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib, schedule="pipelined",
            copy_kernel="copyBuffer", busy_dir=None) -> dict:
    kernel = KERNEL_NAMES.get(schedule, "gemm_" + schedule)
    copy_bytes = copy_mib * 2 ** 20
    cf = counters([copy_fetch_dir], copy_kernel)
    cw = counters([copy_write_dir], copy_kernel)
    if not cf or not cw:
        raise RuntimeError("copy kernel not found in the calibration runs")
    fetch_kib_copy = next(iter(cf.values()))["FETCH_SIZE"]
    write_kib_copy = next(iter(cw.values()))["WRITE_SIZE"]
    f_scale = copy_bytes / (fetch_kib_copy * 1024)
    w_scale = copy_bytes / (write_kib_copy * 1024)
    g_f = next(iter(counters([fetch_dir], kernel).values()))
    g_w = next(iter(counters([write_dir], kernel).values()))
    fetch = g_f["FETCH_SIZE"] * 1024 * f_scale
    write = g_w["WRITE_SIZE"] * 1024 * w_scale
    r = {"fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
         "hbm_bytes_per_launch": round(fetch + write), "fetch_scale": round(f_scale, 5),
         "write_scale": round(w_scale, 5), "copy_calibration_mib": copy_mib,
         "kernel_code_sha256": kernel_code_hash(schedule)}
    if busy_dir:
        ag = agent(busy_dir)
        cs = next(iter(counters([busy_dir], kernel).values()))
        d = derived(cs, int(ag.get("Num_Xcc", 8)), int(ag.get("Simd_Count", 1024)))
        r["mfma_busy"] = round(d["mfma_busy"], 4)
        r["clock_GHz"] = round(d["clock_GHz"], 3)
    return r


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--kernel", default="")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", default="")
    t = sub.add_parser("traffic")
    for f in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + f.replace("_", "-"), required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--schedule", default="pipelined", choices=sorted(KERNEL_SOURCES))
    t.add_argument("--update", default=None, help="JSON file to add the result to")
    t.add_argument("--busy", default=None, help="counter run with GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES")
    a = ap.parse_args(argv)

    if a.cmd == "stats":
        print("| kernel | calls | avg us | min us | max us |\n|---|---|---|---|---|")
        for k in kernel_stats(a.dir, a.kernel):
            print(f"| `{k['name']}` | {k['calls']} | {k['avg_ns'] / 1e3:.2f} | {k['min_ns'] / 1e3:.2f} | "
                  f"{k['max_ns'] / 1e3:.2f} |")
    elif a.cmd == "counters":
        ag = agent(a.dirs[0])
        n_xcc, simds = int(ag.get("Num_Xcc", 8)), int(ag.get("Simd_Count", 1024))
        for k, cs in counters(a.dirs, a.kernel).items():
            print(f"kernel: `{k}` ({cs['_dispatches']} dispatches, mean duration "
                  f"{cs['_duration_ns'] / 1e3:.2f} us under counter collection)\n")
            print("| counter | mean per dispatch |\n|---|---|")
            for n, v in sorted(cs.items()):
                if not n.startswith("_"):
                    print(f"| {n} | {v:.6g} |")
            for n, v in derived(cs, n_xcc, simds).items():
                print(f"| (derived) {n} | {v:.6g} |")
            print()
    elif a.cmd == "traffic":
        r = traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_mib, a.schedule, busy_dir=a.busy)
        print(json.dumps(r, indent=1))
        if a.update:
            data = {}
            if os.path.exists(a.update):
                data = json.load(open(a.update))
            data[traffic_key(a.workload, a.schedule)] = r
            with open(a.update, "w") as f:
                json.dump(data, f, indent=1, sort_keys=True)
                f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
