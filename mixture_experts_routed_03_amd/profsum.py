"""Condense rocprofv3 CSV output of one bench workload into a short text
summary (per-kernel dispatch durations plus HBM bytes per dispatch from
FETCH_SIZE and WRITE_SIZE, scaled by what the same counters read for a plain
device copy of known size) with a machine-readable block that bench.py reads
back.

    python -m mixture_experts_routed_03_amd.profsum NAME TITLE KT_DIR FETCH_DIR WRITE_DIR \
        "KERNEL-TRACE COMMAND" "PMC COMMAND" [PROBE_MIB]

KT_DIR holds ``run_kernel_trace.csv`` (optionally gzipped, optionally cut down
to the library's kernels) and ``run_kernel_stats.csv`` of a ``--kernel-trace
--stats`` run; FETCH_DIR and WRITE_DIR hold ``run_counter_collection.csv`` of
one ``--pmc`` run each.  The copy probe (``bench.py --copy-probe-mb``) is the
``__amd_rocclr_copyBuffer`` dispatch with the largest counter value.
Writes ``profiles/NAME.md``.

Dispatches that did no work (a replay kernel of a layer that saved its state
exits at once; so does the hot-expert kernel of a call without hot experts)
are left out of the averages: a dispatch counts as working when it took at
least a tenth of the longest dispatch of the same kernel, or moved at least
1% of its largest dispatch's bytes.  rocprofv3's own per-kernel averages
(which include them) are shown beside.
"""

from __future__ import annotations

import collections
import csv
import gzip
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")


def short(n: str) -> str:
    n = n.replace("void ", "")
    return n.split("(")[0] if ("moe::" in n or "rocclr" in n) else n[:60]


def strip_comments(text: str) -> str:
    """C/C++ source without comments and with each run of whitespace folded
    to one space (string and character literals are kept as they are)."""
    out = []
    i, n = 0, len(text)
    while i < n:
        c = text[i]
        if c == "/" and i + 1 < n and text[i + 1] == "/":
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif c == "/" and i + 1 < n and text[i + 1] == "*":
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def code_hash(path: str) -> str:
    """Hash of a source file's code (comments and layout ignored), so that a
    summary stays valid across comment-only edits and goes stale on any
    change to what compiles."""
    with open(path, encoding="utf-8") as fh:
        return hashlib.sha256(strip_comments(fh.read()).encode()).hexdigest()[:16]


def source_hashes(files=None):
    names = sorted(os.listdir(CSRC)) if files is None else files
    return {f: code_hash(os.path.join(CSRC, f)) for f in names}


def _open(path):
    if os.path.exists(path):
        return open(path, newline="")
    return gzip.open(path + ".gz", "rt", newline="")


def read_pmc(d):
    out = collections.defaultdict(list)
    with _open(os.path.join(d, "run_counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            out[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return out


def read_trace(d):
    """{kernel: [dispatch durations in ns, in dispatch order]} of the library's kernels."""
    out = collections.defaultdict(list)
    path = os.path.join(d, "run_kernel_trace.csv")
    if not (os.path.exists(path) or os.path.exists(path + ".gz")):
        return None
    with _open(path) as fh:
        rows = sorted(csv.DictReader(fh), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        k = short(r["Kernel_Name"])
        if "moe::" in k:
            out[k].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def working(durs):
    top = max(durs) if durs else 0
    return [d for d in durs if d >= 0.1 * top]


def main(argv):
    name, title, kt_dir, fetch_dir, write_dir, cmd_kt, cmd_pmc = argv[:7]
    probe_mib = int(argv[7]) if len(argv) > 7 else 1024
    with _open(os.path.join(kt_dir, "run_kernel_stats.csv")) as fh:
        stats = list(csv.DictReader(fh))
    trace = read_trace(kt_dir)
    F, W = read_pmc(fetch_dir), read_pmc(write_dir)
    probe = [k for k in F if "rocclr_copyBuffer" in k]
    probe_bytes = probe_mib * (1 << 20)
    fmax = max(max(F[k]) for k in probe)
    wmax = max(max(W[k]) for k in probe if k in W)
    f_scale = probe_bytes / (fmax * 1024)
    w_scale = probe_bytes / (wmax * 1024)
    lines = [f"# rocprofv3 summary: {name}", "", title, "",
             "Commands (run from the repository root on the GPU box; the summary is",
             "written by `python -m mixture_experts_routed_03_amd.profsum`):", "",
             f"    {cmd_kt}", f"    {cmd_pmc}", "",
             "## Kernel stats", "",
             "Working dispatches: those that took at least a tenth of the kernel's longest "
             "dispatch (replay launches of a layer that saved its state, and hot-expert "
             "launches of a call without hot experts, exit at once).  rocprofv3's own average "
             "over all dispatches is shown beside.", "",
             "| kernel | working / all dispatches | avg us (working) | avg us (all) | total % |",
             "|---|---:|---:|---:|---:|"]
    avg_working = {}
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        n = short(r["Name"])
        if "moe::" not in n and float(r["Percentage"]) < 1.0:
            continue
        wk, cell_w, cell_n = None, "", r["Calls"]
        if trace is not None and n in trace:
            wk = working(trace[n])
            avg_working[n] = round(sum(wk) / len(wk) / 1e3, 2)
            cell_w = f"{avg_working[n]:.1f}"
            cell_n = f"{len(wk)} / {len(trace[n])}"
        lines.append(f"| `{n}` | {cell_n} | {cell_w} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    lines += ["", "## HBM traffic per dispatch (FETCH_SIZE, WRITE_SIZE)", "",
              f"Calibration: one plain {probe_mib} MiB device copy reads FETCH_SIZE = {fmax:.0f} KiB "
              f"and writes WRITE_SIZE = {wmax:.0f} KiB, so FETCH_SIZE is scaled by {f_scale:.3f} "
              f"and WRITE_SIZE by {w_scale:.3f} to get bytes.  Mean over the dispatches of each "
              f"kernel that moved at least 1% of its largest dispatch's bytes (the others exit "
              f"at once, as above).", "",
              "| kernel | dispatches | read GB | write GB |", "|---|---:|---:|---:|"]
    traffic = {}
    for k in sorted(F):
        if "moe::" not in k:
            continue
        fl, wl = F[k], W.get(k, [0.0] * len(F[k]))
        if len(wl) != len(fl):
            wl = [sum(wl) / len(wl)] * len(fl)
        tot = [f * f_scale + w * w_scale for f, w in zip(fl, wl)]
        big = [i for i, t in enumerate(tot) if t >= 0.01 * max(tot)]
        fv = sum(fl[i] for i in big) / len(big) * 1024 * f_scale
        wv = sum(wl[i] for i in big) / len(big) * 1024 * w_scale
        if fv + wv < 1e6:
            continue
        lines.append(f"| `{k}` | {len(big)} of {len(fl)} | {fv / 1e9:.3f} | {wv / 1e9:.3f} |")
        traffic[k] = [round(fv + wv)]
    lines += ["", "Machine-readable (bytes per working dispatch, average working-dispatch "
              "duration; hashes of the kernels' code, comments ignored):",
              "", "```json",
              json.dumps({"traffic_bytes": traffic, "avg_us_working": avg_working,
                          "src_code_sha256_16": source_hashes(),
                          "fetch_scale": f_scale, "write_scale": w_scale}),
              "```", ""]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main(sys.argv[1:])
