"""Turns rocprofv3 databases of bench.py runs into the text summaries under profiles/.

Input: a directory holding, per workload W, the output directories of these runs (each run's
rocpd database `*.db` inside), all taken from the repository root with TMPDIR=/tmp:

  prof_trace_W             rocprofv3 --kernel-trace --stats -d <dir>/prof_trace_W -o run --
                               python3 bench.py --extra none --no-cpu-baseline --steps 10
                               --warmup 3 --workload W
  prof_pmc_FETCH_SIZE_W    rocprofv3 --pmc FETCH_SIZE -d <dir>/prof_pmc_FETCH_SIZE_W -o run --
                               python3 bench.py ... --workload W --calibrate-copy-mb 512
  prof_pmc_WRITE_SIZE_W    the same with --pmc WRITE_SIZE

Output: profiles/kernels_W.md for every traced workload and, for the workloads with counter
runs, profiles/traffic_decode_prefill_mxfp8.md and profiles/traffic.json. bench.py reads the
latter for its roofline `traffic` figure, keyed by the sha256 of the GEMM source the counters
were taken on.

Usage: python profile_summary.py <dir> [--traffic W=KERNEL ...] [--out DIR (default profiles/)]
"""
import argparse
import glob
import hashlib
import json
import os
import sqlite3

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
LOADTIME = ("k_quant_canonical", "k_prepack")  # weight preparation, not part of a forward call
TRACE_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -d <out> -o run -- "
             "python3 bench.py --extra none --no-cpu-baseline --steps 10 --warmup 3 --workload {wl}")
PMC_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} -d <out> -o run -- python3 bench.py "
           "--extra none --no-cpu-baseline --steps 10 --warmup 3 --workload {wl} "
           "--calibrate-copy-mb 512")


def short(name):
    n = name.replace("void ", "", 1).replace("mxmoe::(anonymous namespace)::", "")
    i = n.find(">(")
    return n[:i + 1] if i >= 0 else n.split("(")[0]


def ours(name):
    return name.startswith("void mxmoe::") or name.startswith("mxmoe::")


def database(d):
    found = glob.glob(os.path.join(d, "*.db"))
    if len(found) != 1:
        raise SystemExit(f"expected one rocpd database in {d}, found {len(found)}")
    return found[0]


def kernels(db):
    c = sqlite3.connect(db)
    rows = c.execute("select name, duration, grid_x*grid_y*grid_z, "
                     "workgroup_x*workgroup_y*workgroup_z, lds_size from kernels").fetchall()
    d = {}
    for name, dur, grid, wg, lds in rows:
        if not ours(name) or short(name).startswith(LOADTIME):
            continue
        d.setdefault(short(name), {"dur": [], "grid": grid, "wg": wg, "lds": lds})["dur"].append(dur / 1e3)
    return d


def trace_md(src, wl, out):
    d = kernels(database(os.path.join(src, f"prof_trace_{wl}")))
    lines = [f"# Kernel durations: {wl}", "", "Command (repository root on the MI355X box):", "", "```",
             TRACE_CMD.format(wl=wl), "```", "",
             "bench.py runs 3 warm-up and 10 timed forward calls, a stage-event pass of 10 and, at "
             "decode sizes, the same calls replayed from HIP graphs (3 + 10); weights rotate over "
             "several device copies, so each call streams its expert weights from HBM.",
             "Durations from the rocprofv3 kernel trace (rocpd database, `kernels` view), "
             "microseconds per launch, summarised by `profile_summary.py`. Load-time kernels "
             "(weight quantisation, prepack) and torch's own kernels are left out.", "",
             "| kernel | launches | avg us | min us | max us | grid threads | workgroup | LDS bytes |",
             "|---|---|---|---|---|---|---|---|"]
    tot = 0.0
    for s, v in sorted(d.items(), key=lambda kv: -np.mean(kv[1]["dur"])):
        a = np.mean(v["dur"])
        if not s.startswith("k_gate"):
            tot += a
        lines.append(f"| `{s}` | {len(v['dur'])} | {a:.2f} | {min(v['dur']):.2f} | "
                     f"{max(v['dur']):.2f} | {v['grid']} | {v['wg']} | {v['lds']} |")
    lines += ["", f"Sum of the per-launch averages of the block's kernels: {tot:.1f} us per forward call.",
              "`k_gate` (and `k_gate_lds`) is the router gate in front of the block (bench.py's "
              "`gate` timing, weights in cache), not part of that sum."]
    with open(os.path.join(out, f"kernels_{wl}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return d


def pmc(db, counter):
    c = sqlite3.connect(db)
    rows = c.execute("select kernel_name, grid_size, value from counters_collection "
                     "where counter_name=? order by id", (counter,)).fetchall()
    d, copies = {}, []
    for name, _, val in rows:
        if name.startswith("__amd_rocclr_copyBuffer"):
            copies.append(val)
        elif ours(name) and not short(name).startswith(LOADTIME):
            d.setdefault(short(name), []).append(val)
    return d, copies


def traffic(src, gate_up, out):
    """gate_up: workload -> name of its gate_up kernel in the trace."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "gemm_dev.h", "device.h"):   # bench.py's GEMM_SOURCES, same order
        h.update(open(os.path.join(ROOT, "mx_quantized_grouped_amd", "csrc", f), "rb").read())
    sha = h.hexdigest()[:16]
    rec = {}
    md = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
          "Two counter runs per workload, one counter each (FETCH_SIZE, then WRITE_SIZE), "
          "summarised by `profile_summary.py`:", ""]
    for wl, gk in gate_up.items():
        f, fc = pmc(database(os.path.join(src, f"prof_pmc_FETCH_SIZE_{wl}")), "FETCH_SIZE")
        w, wc = pmc(database(os.path.join(src, f"prof_pmc_WRITE_SIZE_{wl}")), "WRITE_SIZE")
        # bench.py --calibrate-copy-mb 512 runs three 512 MiB device copies before anything else
        fcopy, wcopy = np.mean(fc[:3]), np.mean(wc[:3])
        kib = 512 * 1024
        fs, ws = kib / fcopy, kib / wcopy
        tr = kernels(database(os.path.join(src, f"prof_trace_{wl}")))
        md += ["```", PMC_CMD.format(c="FETCH_SIZE", wl=wl), PMC_CMD.format(c="WRITE_SIZE", wl=wl),
               "```", "",
               f"Calibration ({wl} runs): a 512 MiB device-to-device copy (3 launches) reads "
               f"{fcopy:.0f} KiB by FETCH_SIZE and writes {wcopy:.0f} KiB by WRITE_SIZE, against "
               f"524288 KiB each: scale factors {fs:.3f} (fetch) and {ws:.3f} (write).", "",
               f"## {wl}", "",
               "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB | avg us (kernel trace) |",
               "|---|---|---|---|---|---|"]
        for s in sorted(f, key=lambda k: -np.mean(f[k])):
            fv, wv = np.mean(f[s]), np.mean(w.get(s, [0]))
            us = np.mean(tr[s]["dur"]) if s in tr else float("nan")
            md.append(f"| `{s}` | {fv:.0f} | {wv:.0f} | {fv * fs * 1024 / 1e6:.1f} | "
                      f"{wv * ws * 1024 / 1e6:.1f} | {us:.2f} |")
        rb, wb = np.mean(f[gk]) * fs * 1024, np.mean(w[gk]) * ws * 1024
        md += ["", f"gate_up (`{gk}`): {(rb + wb) / 1e6:.1f} MB of HBM traffic per launch.", ""]
        rec[wl] = {"kernel": gk, "gemm_src_sha": sha, "bytes_per_launch": rb + wb, "read_bytes": rb,
                   "write_bytes": wb, "fetch_scale": fs, "write_scale": ws}
    with open(os.path.join(out, "traffic_decode_prefill_mxfp8.md"), "w") as f:
        f.write("\n".join(md))
    with open(os.path.join(out, "traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    return rec


MFMA_CMD = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES "
            "GRBM_GUI_ACTIVE -d <out> -o run -- python3 bench.py --extra none --no-cpu-baseline "
            "--steps 10 --warmup 3 --workload {wl}")


def mfma_util(src, wls, out):
    """MFMA busy fraction per kernel from prof_mfma_W runs: SQ_VALU_MFMA_BUSY_CYCLES (per SIMD,
    summed over all SIMDs) over the launch's SIMD-cycles, GRBM_GUI_ACTIVE (summed over the 8
    XCDs, so / 8 for the GPU's busy cycles) times 1024 SIMDs (256 CUs x 4)."""
    md = ["# MFMA utilisation of the large-M GEMMs (rocprofv3 counters)", "",
          "One counter run per workload (rocpd database, `counters_collection` view, one value per "
          "dispatch and counter, summed over the counter's instances). Per launch: "
          "SQ_VALU_MFMA_BUSY_CYCLES (a per-SIMD count, summed over all SIMDs) divided by the "
          "SIMD-cycles of the launch, i.e. GRBM_GUI_ACTIVE (summed over the 8 XCDs, so divided by 8 "
          "for the GPU's busy cycles) times 1024 SIMDs (256 CUs x 4). Summarised by "
          "`profile_summary.py --mfma`.", "", "Commands (repository root on the MI355X box):", "",
          "```"] + [MFMA_CMD.format(wl=wl) for wl in wls] + ["```", "",
          "| workload | kernel | launches | MFMA busy (% of SIMD-cycles) |", "|---|---|---|---|"]
    res = {}
    for wl in wls:
        c = sqlite3.connect(database(os.path.join(src, f"prof_mfma_{wl}")))
        rows = c.execute("select dispatch_id, kernel_name, counter_name, sum(value) from "
                         "counters_collection group by dispatch_id, counter_name").fetchall()
        disp = {}
        for d, name, ctr, val in rows:
            disp.setdefault(d, [name, {}])[1][ctr] = val
        per = {}
        for name, v in disp.values():
            if not ours(name) or short(name).startswith(LOADTIME):
                continue
            if not short(name).startswith(("k_gemm_tile", "k_gemm_direct", "k_gate")):
                continue
            busy, act = v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), v.get("GRBM_GUI_ACTIVE", 0.0)
            if act > 0:
                per.setdefault(short(name), []).append(busy / (act / 8 * 1024))
        for k in sorted(per, key=lambda k: -np.mean(per[k])):
            md.append(f"| {wl} | `{k}` | {len(per[k])} | {100 * np.mean(per[k]):.1f} |")
            res[(wl, k)] = float(np.mean(per[k]))
    md += ["", "`k_gate` is the router gate in front of the block (bf16 MFMA). For launches of a few tens "
           "of microseconds (the gate) GRBM_GUI_ACTIVE covers more than the kernel, so their fraction "
           "reads low. The busy count includes the padding rows each tile multiplies."]
    with open(os.path.join(out, "mfma_util_prefill.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("src", help="directory with the prof_trace_* / prof_pmc_* run outputs")
    ap.add_argument("--traffic", nargs="*", default=[
        "decode_mxfp8=k_gemm_stream<0, 1, true, 3, 1, 2, true, 1>",
        "prefill_mxfp8=k_gemm_tile<0, true, true, true>"],
        help="WORKLOAD=gate_up kernel name, for the counter summary")
    ap.add_argument("--mfma", nargs="*", default=[],
                    help="workloads with prof_mfma_W counter runs, for mfma_util_prefill.md")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args(argv)
    for d in sorted(glob.glob(os.path.join(a.src, "prof_trace_*"))):
        if os.path.isdir(d):
            wl = os.path.basename(d)[len("prof_trace_"):]
            t = trace_md(a.src, wl, a.out)
            print(wl, {k: round(float(np.mean(v["dur"])), 2) for k, v in t.items()})
    if a.traffic:
        print(json.dumps(traffic(a.src, dict(x.split("=", 1) for x in a.traffic), a.out), indent=1))
    if a.mfma:
        for (wl, k), v in mfma_util(a.src, a.mfma, a.out).items():
            print(wl, k, round(100 * v, 1))


if __name__ == "__main__":
    main()
