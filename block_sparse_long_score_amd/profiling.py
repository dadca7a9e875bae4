"""Turns rocprofv3 output into the figures bench.py reports.

    python -m block_sparse_long_score_amd.profiling stats DIR
        Markdown table of a `rocprofv3 --kernel-trace --stats` run (per-kernel
        calls and average / total device time).

    python -m block_sparse_long_score_amd.profiling traffic --kernel NAME --workload W \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N [--out FILE]
        HBM bytes per launch of kernel NAME from two `rocprofv3 --pmc` runs
        (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the
        same counter reads for a plain device copy of N bytes (bench.py
        --copy-calibration).  Merged into FILE (profiles/traffic.json), keyed by
        kernel and workload, with a hash of the kernel's sources: bench.py
        reports the figure only while those sources are unchanged.

    python -m block_sparse_long_score_amd.profiling counters DIR [--kernel NAME ...]
        Markdown table of every counter in a `rocprofv3 --pmc` run: the mean
        value per dispatch (summed over the chip) for each kernel.

Host-side bookkeeping only; nothing here runs on the GPU.
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

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# Sources holding each kernel's device code (launch.h is host-only).
KERNEL_SOURCES = {
    "index_scores_tiled": ["index_score.hip", "msa_device.h"],
    "index_scores_skinny": ["index_score.hip", "msa_device.h"],
    "sparse_kv_outer": ["sparse_attn.hip", "msa_device.h"],
    "merge_partials": ["sparse_attn.hip", "msa_device.h"],
    "sparse_decode_blocks": ["sparse_attn.hip", "msa_device.h"],
    "block_topk_rows": ["block_topk.hip", "msa_select.h", "msa_device.h"],
    "block_topk_wg": ["block_topk.hip", "msa_select.h", "msa_device.h"],
    "dense_prefill": ["dense_attn.hip", "msa_device.h"],
    "index_topk_tiled": ["index_score.hip", "msa_select.h", "msa_device.h"],
    "topk_merge_pieces": ["index_score.hip", "msa_select.h", "msa_device.h"],
}


def kernel_sources_sha256(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    """`void msa::(anonymous namespace)::sparse_kv_outer<128, 3>(...)` -> `sparse_kv_outer`."""
    n = name.replace("msa::(anonymous namespace)::", "").replace("void ", "").strip()
    return n.split("(")[0].split("<")[0].strip()


def _csvs(root: str, pattern: str):
    return sorted(glob.glob(os.path.join(root, "**", pattern), recursive=True))


def counter_per_dispatch(root: str, counter: str) -> dict:
    """{kernel short name: (mean counter value per dispatch, dispatches)}."""
    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    for f in _csvs(root, "*counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                k = short_name(r["Kernel_Name"])
                tot[k] += float(r["Counter_Value"])
                disp[k].add(r["Dispatch_Id"])
    return {k: (tot[k] / len(disp[k]), len(disp[k])) for k in tot}


def kernel_stats(root: str) -> list:
    rows = []
    for f in _csvs(root, "*kernel_stats.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((short_name(r["Name"]), r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e6,
                             float(r["TotalDurationNs"]) / 1e6))
    return sorted(rows, key=lambda x: -x[4])


def cmd_stats(a) -> None:
    print("| kernel | calls | avg ms | total ms |")
    print("|---|---:|---:|---:|")
    for short, full, calls, avg, tot in kernel_stats(a.dir):
        label = full.replace("msa::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        print(f"| `{label}` | {calls} | {avg:.3f} | {tot:.3f} |")


def _copy_value(root: str, counter: str) -> float:
    vals = {k: v for k, v in counter_per_dispatch(root, counter).items() if "copyBuffer" in k or "copy" in k.lower()}
    if not vals:
        raise SystemExit(f"no copy kernel found under {root}")
    # the calibration run's copy is its largest-volume copy
    return max(v for v, _ in vals.values())


def cmd_traffic(a) -> None:
    fetch = counter_per_dispatch(a.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(a.write, "WRITE_SIZE")
    if a.kernel not in fetch or a.kernel not in write:
        raise SystemExit(f"{a.kernel} not found (fetch: {sorted(fetch)}, write: {sorted(write)})")
    cf = _copy_value(a.copy_fetch, "FETCH_SIZE") * 1024.0
    cw = _copy_value(a.copy_write, "WRITE_SIZE") * 1024.0
    ff, fw = a.copy_bytes / cf, a.copy_bytes / cw
    entry = {
        "read_bytes": fetch[a.kernel][0] * 1024.0 * ff,
        "write_bytes": write[a.kernel][0] * 1024.0 * fw,
        "fetch_kib_per_dispatch": fetch[a.kernel][0],
        "write_kib_per_dispatch": write[a.kernel][0],
        "dispatches": [fetch[a.kernel][1], write[a.kernel][1]],
        "copy_bytes": a.copy_bytes,
        "fetch_scale": ff,
        "write_scale": fw,
        "sources_sha256": kernel_sources_sha256(a.kernel),
    }
    rec = {}
    if a.out and os.path.exists(a.out):
        with open(a.out) as fh:
            rec = json.load(fh)
    rec.setdefault(a.kernel, {})[a.workload] = entry
    text = json.dumps(rec, indent=2, sort_keys=True)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text + "\n")
    print(json.dumps({a.kernel: {a.workload: entry}}, indent=2))


def cmd_counters(a) -> None:
    names = set()
    for f in _csvs(a.dir, "*counter_collection.csv"):
        with open(f) as fh:
            names.update(r["Counter_Name"] for r in csv.DictReader(fh))
    per = {n: counter_per_dispatch(a.dir, n) for n in sorted(names)}
    kernels = sorted({k for v in per.values() for k in v})
    if a.kernel:
        kernels = [k for k in kernels if k in a.kernel]
    print("| kernel | dispatches | " + " | ".join(sorted(names)) + " |")
    print("|---|---:|" + "---:|" * len(names))
    for k in kernels:
        disp = max(per[n][k][1] for n in per if k in per[n])
        vals = [f"{per[n][k][0]:.4g}" if k in per[n] else "-" for n in sorted(names)]
        print(f"| `{k}` | {disp} | " + " | ".join(vals) + " |")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m block_sparse_long_score_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--out")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--kernel", nargs="*")
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
