"""Condense rocprofv3 CSV output of one bench workload into a short text
summary (kernel stats plus HBM bytes per dispatch from FETCH_SIZE and
WRITE_SIZE, scaled by what the same counters read for a plain device copy of
known size) with a machine-readable block that bench.py reads back.

    python -m mixture_experts_routed_03_amd.profsum NAME TITLE KT_DIR FETCH_DIR WRITE_DIR \
        "KERNEL-TRACE COMMAND" "PMC COMMAND" [PROBE_MIB]

KT_DIR holds ``run_kernel_stats.csv`` of a ``--kernel-trace --stats`` run;
FETCH_DIR and WRITE_DIR hold ``run_counter_collection.csv`` of one ``--pmc``
run each.  The copy probe (``bench.py --copy-probe-mb``) is the
``__amd_rocclr_copyBuffer`` dispatch with the largest counter value.
Writes ``profiles/NAME.md``.
"""

from __future__ import annotations

import collections
import csv
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


def read_pmc(d):
    out = collections.defaultdict(list)
    with open(os.path.join(d, "run_counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            out[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return out


def source_hashes():
    out = {}
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            out[f] = hashlib.sha256(fh.read()).hexdigest()[:16]
    return out


def main(argv):
    name, title, kt_dir, fetch_dir, write_dir, cmd_kt, cmd_pmc = argv[:7]
    probe_mib = int(argv[7]) if len(argv) > 7 else 1024
    with open(os.path.join(kt_dir, "run_kernel_stats.csv")) as fh:
        stats = list(csv.DictReader(fh))
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
             "## Kernel stats", "", "| kernel | calls | avg us | total % |",
             "|---|---:|---:|---:|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        n = short(r["Name"])
        if "moe::" not in n and float(r["Percentage"]) < 1.0:
            continue
        lines.append(f"| `{n}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    lines += ["", "## HBM traffic per dispatch (FETCH_SIZE, WRITE_SIZE)", "",
              f"Calibration: one plain {probe_mib} MiB device copy reads FETCH_SIZE = {fmax:.0f} KiB "
              f"and writes WRITE_SIZE = {wmax:.0f} KiB, so FETCH_SIZE is scaled by {f_scale:.3f} "
              f"and WRITE_SIZE by {w_scale:.3f} to get bytes.  Mean over the dispatches of each "
              f"kernel that moved at least 1% of its largest dispatch's bytes (the others are "
              f"replay launches that exit at once; the kernel-stats averages above include "
              f"them).", "",
              "| kernel | dispatches | read GB | write GB |", "|---|---:|---:|---:|"]
    traffic = {}
    for k in sorted(F):
        if "moe::" not in k:
            continue
        fl, wl = F[k], W.get(k, [0.0] * len(F[k]))
        if len(wl) != len(fl):
            wl = [sum(wl) / len(wl)] * len(fl)
        tot = [f * f_scale + w * w_scale for f, w in zip(fl, wl)]
        # dispatches that exit at once (a replay kernel of a layer that saved
        # its state) are left out of the mean
        big = [i for i, t in enumerate(tot) if t >= 0.01 * max(tot)]
        fv = sum(fl[i] for i in big) / len(big) * 1024 * f_scale
        wv = sum(wl[i] for i in big) / len(big) * 1024 * w_scale
        if fv + wv < 1e6:
            continue
        lines.append(f"| `{k}` | {len(big)} of {len(fl)} | {fv / 1e9:.3f} | {wv / 1e9:.3f} |")
        traffic[k] = [round(fv + wv)]
    lines += ["", "Machine-readable (bytes per dispatch; source hashes of the kernels measured):",
              "", "```json",
              json.dumps({"traffic_bytes": traffic, "src_sha256_16": source_hashes(),
                          "fetch_scale": f_scale, "write_scale": w_scale}),
              "```", ""]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main(sys.argv[1:])
