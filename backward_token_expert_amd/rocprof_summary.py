"""Summaries of rocprofv3 output for liblrm's kernels (markdown, a few KB).

  python -m backward_token_expert_amd.rocprof_summary stats KERNEL_STATS_CSV --title T --command C
  python -m backward_token_expert_amd.rocprof_summary counters PMC_ROOT --copy-bytes N \
      --workload W --title T --command C

`counters` reads the pass directories PMC_ROOT/p*/ (one rocprofv3 --pmc run each; a run holds
`*_counter_collection.csv`).  HBM traffic comes from FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
each scaled by the factor that makes the same counter, read on a plain copy of N bytes (the largest
`__amd_rocclr_copyBuffer` dispatch of the run), equal N.  The output ends with a `traffic-record:`
line (JSON) holding, for the GEMM entry points, the calibrated bytes per launch and a digest of the
sources the kernel is built from; bench.py reports that traffic only while the digest still matches
the tree, so a changed kernel reports null until its counters are taken again.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# C-ABI entry point -> (pattern of its GEMM kernels' short names, translation unit).  The one-launch
# GEMMs are two launches of gemm_fused (last template argument 0 and 1: one of them runs the
# product, the other returns at once or adds split experts' partial sums), whose counters are
# summed; the argument before it tells FC2's launches (2) from FC1's (1).
GEMM_KERNELS = {"lrm_grouped_dw": (r"(dw_bf16|dw_f32)\b", "gemm.hip"),
                "lrm_grouped_dx": (r"(dx_bf16|dx_f32)\b", "gemm.hip"),
                "lrm_grouped_dw_dx": (r"gemm_fused<.*, 2, [01]>$", "gemm.hip"),
                "lrm_grouped_fc1_dw_dx": (r"gemm_fused<.*, 1, [01]>$", "gemm.hip")}
_SHARED = ("lrm_device.hpp", "lrm_internal.hpp")


def _without_profiling_blocks(text: str) -> str:
    """Drop `#ifdef LRM_TIMELINE ... #endif` blocks (nesting-aware): they exist only in the
    profiling build, so they do not change the kernels the counters were taken on."""
    out, depth = [], 0
    for line in text.splitlines():
        t = line.strip()
        if depth == 0 and t.startswith("#ifdef LRM_TIMELINE"):
            depth = 1
            continue
        if depth > 0:
            if t.startswith("#if"):
                depth += 1
            elif t.startswith("#endif"):
                depth -= 1
            continue
        out.append(line)
    return "\n".join(out)


def _code_only(text: str) -> str:
    """Source text without comments, blank space and profiling-build blocks, so that comment
    edits and timeline instrumentation keep the digest."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = _without_profiling_blocks(text)
    return " ".join(text.split())


def source_digest(call: str) -> str:
    """sha256 over the code (comments dropped) of the sources and build flags the kernel of C-ABI
    entry `call` is built from."""
    tu = GEMM_KERNELS[call][1]
    h = hashlib.sha256()
    for f in (os.path.join(CSRC, tu), *(os.path.join(CSRC, s) for s in _SHARED),
              os.path.join(PKG, "build.py")):
        with open(f, encoding="utf-8") as fh:
            code = fh.read() if f.endswith(".py") else _code_only(fh.read())
        h.update(os.path.basename(f).encode() + b"\0" + code.encode())
    return h.hexdigest()


def short_name(n: str) -> str:
    n = n.replace("lrm::(anonymous namespace)::", "").replace("void ", "")
    return re.sub(r"\(.*", "", n)[:90]


def stats_table(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg µs | min µs | max µs | total ms | % |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out)


def read_counters(root: str):
    """{kernel: {counter: [per-dispatch values]}} and {kernel: {counter: [per-dispatch durations
    (ns) of the dispatches that counter was read on]}}."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(lambda: collections.defaultdict(list))
    for f in sorted(glob.glob(os.path.join(root, "p*", "*counter_collection.csv"))):
        for r in csv.DictReader(open(f)):
            n = short_name(r["Kernel_Name"])
            vals[n][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if "Start_Timestamp" in r:
                durs[n][r["Counter_Name"]].append(
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return vals, durs


def copy_scales(vals, copy_bytes: int):
    cp = vals.get("__amd_rocclr_copyBuffer", {})
    fetch = max(cp.get("FETCH_SIZE", [0.0]))
    write = max(cp.get("WRITE_SIZE", [0.0]))
    if fetch <= 0 or write <= 0:
        raise SystemExit("no copy-kernel FETCH_SIZE/WRITE_SIZE found for calibration")
    return copy_bytes / (fetch * 1024), copy_bytes / (write * 1024), fetch, write


def counters_report(root: str, copy_bytes: int, workload: str):
    vals, durs = read_counters(root)
    fs, ws, cf, cw = copy_scales(vals, copy_bytes)
    lines = [f"Copy calibration: a {copy_bytes} B copy reads FETCH_SIZE {cf:.0f} KiB and "
             f"WRITE_SIZE {cw:.0f} KiB, so FETCH_SIZE x {fs:.3f} and WRITE_SIZE x {ws:.3f} give "
             "bytes.", "",
             "Clock: GRBM_GUI_ACTIVE (GPU cycles, summed over the 8 XCDs) / 8 / the dispatch's "
             "duration.", "",
             "| kernel | dispatches | clock MHz | MFMA busy % | wait-inst % | L2 hit % | "
             "LDS bank conflicts | FETCH KiB | WRITE KiB | HBM MB (calibrated) |",
             "|---|---|---|---|---|---|---|---|---|---|"]

    def avg(d, c):
        v = d.get(c)
        return sum(v) / len(v) if v else None

    rec = {"workload": workload, "fetch_scale": fs, "write_scale": ws, "kernels": {}}
    order = sorted(vals, key=lambda k: -(avg(vals[k], "GRBM_GUI_ACTIVE") or 0))
    for k in order:
        if k.startswith("at::") or k.startswith("__amd"):
            continue
        d = vals[k]
        gui = avg(d, "GRBM_GUI_ACTIVE")
        mf = avg(d, "SQ_VALU_MFMA_BUSY_CYCLES")
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs; SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs
        mfp = 100 * mf / (gui / 8 * 1024) if gui and mf is not None else None
        wi, wc = avg(d, "SQ_WAIT_INST_ANY"), avg(d, "SQ_WAVE_CYCLES")
        hit, miss = avg(d, "TCC_HIT_sum"), avg(d, "TCC_MISS_sum")
        fe, wr = avg(d, "FETCH_SIZE"), avg(d, "WRITE_SIZE")
        conf = avg(d, "SQ_LDS_BANK_CONFLICT")
        dd = durs.get(k, {}).get("GRBM_GUI_ACTIVE", [])
        clk = (sum(d["GRBM_GUI_ACTIVE"]) / 8 / sum(dd) * 1e3
               if gui and dd and sum(dd) > 0 else None)
        mb = (fe * 1024 * fs + wr * 1024 * ws) / 1e6 if fe is not None and wr is not None else None
        f = lambda x, p=1: "–" if x is None else f"{x:.{p}f}"
        n = max((len(v) for v in d.values()), default=0)
        lines.append(f"| {k} | {n} | {f(clk, 0)} | {f(mfp)} | "
                     f"{f(100 * wi / wc if wi is not None and wc else None)} | "
                     f"{f(100 * hit / (hit + miss) if hit is not None and miss is not None else None)} | "
                     f"{f(conf, 0)} | {f(fe, 0)} | {f(wr, 0)} | {f(mb)} |")
        for call, (names, _) in GEMM_KERNELS.items():
            if re.match(names, k) and mb is not None:
                r = rec["kernels"].setdefault(call, {"kernels": [], "traffic_bytes": 0.0,
                                                     "fetch_bytes": 0.0, "write_bytes": 0.0,
                                                     "source_sha256": source_digest(call)})
                r["kernels"].append(k)
                r["traffic_bytes"] += mb * 1e6
                r["fetch_bytes"] += fe * 1024 * fs
                r["write_bytes"] += wr * 1024 * ws
                # clock and MFMA busy of the launch that ran the product (the busier one)
                if gui is not None and gui > r.get("_gui", -1.0):
                    r.update({"_gui": gui, "kernel": k, "clock_mhz": clk, "mfma_busy_pct": mfp})
    for r in rec["kernels"].values():
        r.pop("_gui", None)
    return "\n".join(lines), rec


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--title", required=True)
    a.add_argument("--command", required=True)
    b = sub.add_parser("counters")
    b.add_argument("root")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--title", required=True)
    b.add_argument("--command", required=True)
    args = ap.parse_args()
    head = f"# {args.title}\n\nCommand (R = repository root):\n\n```\n{args.command}\n```\n"
    if args.cmd == "stats":
        print(head)
        print(stats_table(args.csv))
    else:
        body, rec = counters_report(args.root, args.copy_bytes, args.workload)
        print(head)
        print(body)
        print()
        print("traffic-record: " + json.dumps(rec, sort_keys=True))


if __name__ == "__main__":
    main()
