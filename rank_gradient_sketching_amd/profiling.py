"""Summaries of rocprofv3 output for the LoGRA kernels.

Two commands, both reading the CSV files rocprofv3 writes with
`--output-format csv`:

  stats    kernel-trace statistics (`*_kernel_stats.csv`) -> markdown table
           of the library's kernels (calls, average / min / max duration).
  traffic  two counter runs (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`,
           `*_counter_collection.csv`) -> HBM bytes per dispatch of each
           kernel, scaled by what the same counters read for a plain device
           copy of known size (the largest dispatch of the hand-written
           `copy_chunks` kernel of liblogra_calib.so in the run).
  mfma     one counter run (`--pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES
           SQ_BUSY_CU_CYCLES SQ_INSTS_VALU`) -> per kernel and grid size: MFMA
           and VALU instructions per dispatch and the matrix-core busy share,
           SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES).

`traffic` also records a hash of the kernel sources, so a consumer can tell
whether the counters still describe the code being run.

Usage:
  python -m rank_gradient_sketching_amd.profiling stats STATS_CSV --out F.md --cmd "..."
  python -m rank_gradient_sketching_amd.profiling traffic FETCH_DIR WRITE_DIR \
      --copy-bytes N --out F.md --cmd "..."
  python -m rank_gradient_sketching_amd.profiling mfma PMC_DIR --out F.md --cmd "..."
"""
import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")


def _code_only(text):
    """C++ source text without comments and with whitespace runs collapsed,
    so that edits to comments do not mark the counters stale (the sources
    hold no string literal that contains a comment marker)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    """sha256 over the code (comments stripped) of the library's HIP / C++
    sources, in name order."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if path.endswith((".hip", ".hpp", ".cpp", ".h")):
            h.update(os.path.basename(path).encode())
            with open(path, encoding="utf-8") as f:
                h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def short_name(name):
    """'void logra::(anonymous namespace)::accumulate_kernel<4, 4, 8, false>(...)'
    -> 'accumulate_kernel<4, 4, 8, false>' (parameter types may name logra:: too)."""
    base = name.replace("(anonymous namespace)::", "")
    if base.startswith("void "):
        base = base[5:]
    depth, out = 0, []
    for ch in base:
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    base = "".join(out).strip()
    if base.startswith("logra::"):
        return base[len("logra::"):]
    return base[:80]


def stats_table(stats_csv):
    rows = []
    for r in csv.DictReader(open(stats_csv)):
        name = r["Name"]
        if "logra" not in name and "copyBuffer" not in name and "copy_chunks" not in name:
            continue
        rows.append(dict(kernel=short_name(name), calls=int(r["Calls"]),
                         avg_us=float(r["AverageNs"]) / 1e3, min_us=float(r["MinNs"]) / 1e3,
                         max_us=float(r["MaxNs"]) / 1e3, pct=float(r["Percentage"])))
    return rows


def counter_per_kernel(run_dir, counter):
    """{kernel: [value per dispatch]} of one counter (KiB for the size counters)."""
    out = collections.defaultdict(list)
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return out


def traffic(fetch_dir, write_dir, copy_bytes):
    fetch = counter_per_kernel(fetch_dir, "FETCH_SIZE")
    write = counter_per_kernel(write_dir, "WRITE_SIZE")
    def is_copy(k):
        return "copyBuffer" in k or "copy_chunks" in k
    cp_f = max((v for k, vs in fetch.items() if is_copy(k) for v in vs), default=None)
    cp_w = max((v for k, vs in write.items() if is_copy(k) for v in vs), default=None)
    if not cp_f or not cp_w:
        raise SystemExit("no copy dispatch (copy_chunks or copyBuffer) found for calibration")
    f_scale = copy_bytes / (cp_f * 1024.0)
    w_scale = copy_bytes / (cp_w * 1024.0)
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        if "logra" in k or k.split("<")[0].endswith("_kernel"):
            fr = statistics.median(fetch[k]) * 1024.0 * f_scale if k in fetch else None
            wr = statistics.median(write[k]) * 1024.0 * w_scale if k in write else None
            kernels[k] = dict(read_bytes=fr, write_bytes=wr,
                              dispatches=max(len(fetch.get(k, [])), len(write.get(k, []))))
    return dict(copy_bytes=copy_bytes, fetch_scale=f_scale, write_scale=w_scale,
                copy_fetch_kib=cp_f, copy_write_kib=cp_w, kernels=kernels,
                source_hash=kernel_source_hash())


MFMA_COUNTERS = ("SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU")
STALL_COUNTERS = ("SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_VALU")


def mfma_table(run_dir, counters=MFMA_COUNTERS):
    """[(kernel, grid, dispatches, {counter: median per dispatch})] of the library's kernels."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if "logra" not in r["Kernel_Name"] or r["Counter_Name"] not in counters:
                continue
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]))
            vals[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    rows = []
    for (kn, grid), cs in sorted(vals.items()):
        med = {c: statistics.median(v) for c, v in cs.items()}
        rows.append((kn, grid, max(len(v) for v in cs.values()), med))
    return rows


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("stats_csv")
    s.add_argument("--out", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="Kernel durations")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("pmc_dir")
    m.add_argument("--out", required=True)
    m.add_argument("--cmd", required=True)
    m.add_argument("--title", default="Matrix-core and VALU counters")
    w = sub.add_parser("stalls")
    w.add_argument("pmc_dir")
    w.add_argument("--out", required=True)
    w.add_argument("--cmd", required=True)
    w.add_argument("--title", default="Where the waves spend their cycles")
    a = ap.parse_args()
    if a.cmd_name == "stalls":
        lines = [f"# {a.title}", "", "Command:", "", "```", a.cmd, "```", "",
                 f"Kernel sources: `{kernel_source_hash()}`", "",
                 "Per dispatch (median over dispatches of the same kernel and grid size). "
                 "Shares per wave are fractions of SQ_WAVE_CYCLES (the cycles the waves were "
                 "alive): waiting for any instruction's operands or resources "
                 "(SQ_WAIT_INST_ANY), issuing VALU, scalar, vector-memory and LDS instructions "
                 "(SQ_ACTIVE_INST_*). VALU busy per SIMD = SQ_ACTIVE_INST_VALU / (4 SIMDs x "
                 "SQ_BUSY_CU_CYCLES), the share of a SIMD's cycles in which some wave on it "
                 "issued VALU work.", "",
                 "| kernel | grid (threads) | dispatches | VALU instr | wait | VALU | scalar | "
                 "vector memory | LDS | VALU busy per SIMD |",
                 "|---|---|---|---|---|---|---|---|---|---|"]
        for kn, grid, n, c in mfma_table(a.pmc_dir, STALL_COUNTERS):
            wc = c.get("SQ_WAVE_CYCLES", 0.0)
            busy = c.get("SQ_BUSY_CU_CYCLES", 0.0)

            def share(name):
                return f"{c.get(name, 0.0) / wc:.3f}" if wc else "-"
            simd = f"{c.get('SQ_ACTIVE_INST_VALU', 0.0) / (4.0 * busy):.3f}" if busy else "-"
            lines.append(f"| `{kn}` | {grid} | {n} | {c.get('SQ_INSTS_VALU', 0.0):.0f} | "
                         f"{share('SQ_WAIT_INST_ANY')} | {share('SQ_ACTIVE_INST_VALU')} | "
                         f"{share('SQ_ACTIVE_INST_SCA')} | {share('SQ_ACTIVE_INST_VMEM')} | "
                         f"{share('SQ_ACTIVE_INST_LDS')} | {simd} |")
        open(a.out, "w").write("\n".join(lines) + "\n")
        return
    if a.cmd_name == "mfma":
        lines = [f"# {a.title}", "", "Command:", "", "```", a.cmd, "```", "",
                 f"Kernel sources: `{kernel_source_hash()}`", "",
                 "Per dispatch (median over dispatches of the same kernel and grid size). "
                 "MFMA busy share = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x SQ_BUSY_CU_CYCLES).", "",
                 "| kernel | grid (threads) | dispatches | MFMA instr | VALU instr | VALU / MFMA | MFMA busy share |",
                 "|---|---|---|---|---|---|---|"]
        for kn, grid, n, c in mfma_table(a.pmc_dir):
            mf = c.get("SQ_INSTS_MFMA", 0.0)
            va = c.get("SQ_INSTS_VALU", 0.0)
            busy = c.get("SQ_BUSY_CU_CYCLES", 0.0)
            share = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4.0 * busy) if busy else 0.0
            ratio = f"{va / mf:.1f}" if mf else "-"
            lines.append(f"| `{kn}` | {grid} | {n} | {mf:.0f} | {va:.0f} | {ratio} | {share:.3f} |")
        open(a.out, "w").write("\n".join(lines) + "\n")
        return
    if a.cmd_name == "stats":
        rows = stats_table(a.stats_csv)
        lines = [f"# {a.title}", "", "Command:", "", "```", a.cmd, "```", "",
                 f"Kernel sources: `{kernel_source_hash()}`", "",
                 "| kernel | calls | avg us | min us | max us | % of GPU time |",
                 "|---|---|---|---|---|---|"]
        for r in rows:
            lines.append(f"| `{r['kernel']}` | {r['calls']} | {r['avg_us']:.2f} | "
                         f"{r['min_us']:.2f} | {r['max_us']:.2f} | {r['pct']:.2f} |")
        open(a.out, "w").write("\n".join(lines) + "\n")
    else:
        tr = traffic(a.fetch_dir, a.write_dir, a.copy_bytes)
        lines = ["# HBM traffic per dispatch (rocprofv3 counters, calibrated)", "",
                 "Commands:", "", "```", a.cmd, "```", "",
                 f"Calibration: a {a.copy_bytes} B device copy read FETCH_SIZE "
                 f"{tr['copy_fetch_kib']:.0f} KiB and WRITE_SIZE {tr['copy_write_kib']:.0f} KiB, "
                 f"so bytes = FETCH_SIZE x 1024 x {tr['fetch_scale']:.3f} and "
                 f"WRITE_SIZE x 1024 x {tr['write_scale']:.3f}.", "",
                 f"Kernel sources: `{tr['source_hash']}`", "",
                 "| kernel | dispatches | read MiB | write MiB |", "|---|---|---|---|"]
        for k, v in tr["kernels"].items():
            rd = "-" if v["read_bytes"] is None else f"{v['read_bytes'] / 2**20:.2f}"
            wr = "-" if v["write_bytes"] is None else f"{v['write_bytes'] / 2**20:.2f}"
            lines.append(f"| `{k}` | {v['dispatches']} | {rd} | {wr} |")
        lines += ["", "<!-- traffic-json: " + json.dumps(tr) + " -->"]
        open(a.out, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
