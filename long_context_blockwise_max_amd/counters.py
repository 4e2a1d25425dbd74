"""HBM traffic per kernel launch from two rocprofv3 counter runs.

rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (two runs of the same
command, one counter each) give, per dispatch, the KiB the L2 fetched from and
wrote to memory.  The command also runs one plain elementwise copy of a known
size (bench.py --calib-copy-mib); its readings fix the scale factor from counter
KiB to bytes that really crossed the memory interface, applied to every kernel.

    python -m long_context_blockwise_max_amd.counters \\
        --fetch <fetch run>/run_counter_collection.csv (or run_results.db) \\
        --write <write run>/run_counter_collection.csv (or run_results.db) \\
        --copy-mib 1024 --workload 128k --out profiles/hbm_traffic.json \\
        --summary profiles/hbm_traffic_128k.md --command "<the rocprofv3 lines>"

The JSON keeps the hash of the attention kernels' code (comments ignored) the counters were
taken on; the benchmark reports the traffic only while that hash still matches.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import sys

KERNELS = ("phase1_kernel", "phase2_kernel", "phase2_prep", "rope_fill", "v_cache_fill",
           "phase1_prefix_list", "phase1_order", "select_clear", "select_df", "select_topk",
           "lse_merge_kernel", "self_append")
COPY_MARK = "neg_kernel"


def short_name(full: str) -> str:
    # the second template argument tells the forms of the attention kernels apart
    # (prefix rows, decode); a third, the wave count, does not
    m = re.search(r"phase([12])_kernel<\s*\d+\s*,\s*(true|false)\b", full)
    if m:
        if m.group(1) == "1":
            return "phase1_kernel_prefix_rows" if m.group(2) == "true" else "phase1_kernel"
        return "phase2_kernel_decode" if m.group(2) == "true" else "phase2_kernel"
    for k in KERNELS:
        if k in full:
            return k
    if COPY_MARK in full:
        return "copy"
    if "reduce_kernel" in full and "sum_functor" in full:
        return "cache_evict_read"       # the read pass that evicts the cache before Phase 2
    if "FillFunctor" in full:
        return "fill"
    return full.split("(")[0][-60:]


def _records(path: str):
    """(dispatch id, kernel name, counter name, value) from a rocprofv3 counter
    collection: the CSV output or the rocpd SQLite database."""
    if path.endswith(".db"):
        import sqlite3
        con = sqlite3.connect(path)
        try:
            yield from con.execute("select dispatch_id, kernel_name, counter_name, value "
                                   "from counters_collection")
        finally:
            con.close()
        return
    with open(path) as fh:
        for r in csv.DictReader(fh):
            yield int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])


def per_dispatch(path: str, counter: str):
    """{short kernel name: [KiB per dispatch, ...]} summed over the counter's instances."""
    acc = collections.defaultdict(float)
    names = {}
    for d, name, cname, value in _records(path):
        if cname != counter:
            continue
        acc[int(d)] += float(value)
        names[int(d)] = short_name(name)
    out = collections.defaultdict(list)
    for d in sorted(acc):
        out[names[d]].append(acc[d])
    return out


def algorithmic_bytes(w, kernel):
    """Bytes a launch must move at least: every operand read once, every result written once."""
    from . import costs as C
    if kernel == "phase1_kernel":
        return C.phase1_kernel_bytes(w.n_blocks, w.block_size, w.sink_size, w.chunk_size, w.k_eff,
                                     w.n_q_heads, w.n_kv_heads, w.head_dim)
    if kernel == "phase2_kernel":
        return C.phase2_kernel_bytes(w.batch, w.n_blocks, w.block_size, w.q_len, w.n_q_heads,
                                     w.n_kv_heads, w.head_dim, True)
    return None


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--out", required=True)
    ap.add_argument("--summary", required=True)
    ap.add_argument("--command", default="")
    a = ap.parse_args(argv)

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import workloads as W

    from .source_hash import kernel_source_hash

    fetch = per_dispatch(a.fetch, "FETCH_SIZE")
    write = per_dispatch(a.write, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("no calibration copy kernel in the counter runs")
    copy_bytes = float(a.copy_mib) * (1 << 20)
    f_scale = copy_bytes / (fetch["copy"][0] * 1024.0)
    w_scale = copy_bytes / (write["copy"][0] * 1024.0)
    w = W.WORKLOADS[a.workload]

    rows = {}
    for k in sorted(set(fetch) & set(write)):
        if k == "copy":
            continue
        fb = sum(fetch[k]) / len(fetch[k]) * 1024.0 * f_scale
        wb = sum(write[k]) / len(write[k]) * 1024.0 * w_scale
        ent = {"fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
               "dispatches": len(fetch[k])}
        alg = algorithmic_bytes(w, k)
        if alg is not None:
            ent["algorithmic_bytes"] = alg
            ent["traffic_over_algorithmic"] = round((fb + wb) / alg, 3)
        rows[k] = ent

    rec = {}
    if os.path.exists(a.out):
        with open(a.out) as fh:
            rec = json.load(fh)
    src = kernel_source_hash()
    if rec.get("source_hash") != src:
        rec = {"kernels": {}}
    rec["source_hash"] = src
    rec.setdefault("calibration", {})[a.workload] = {
        "copy_bytes": copy_bytes, "copy_fetch_kib": fetch["copy"][0],
        "copy_write_kib": write["copy"][0], "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4)}
    rec["kernels"][a.workload] = rows
    rec.setdefault("commands", {})[a.workload] = a.command
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)

    lines = [f"# HBM traffic per launch, {a.workload} workload", "",
             "Command:", "", "```", a.command.strip(), "```", "",
             f"Calibration: one elementwise copy of {a.copy_mib} MiB read "
             f"{fetch['copy'][0]:.0f} KiB (FETCH_SIZE) and wrote {write['copy'][0]:.0f} KiB "
             f"(WRITE_SIZE): scale factors {f_scale:.4f} (fetch), {w_scale:.4f} (write).", "",
             f"Kernel code hash (comments ignored): {src}", "",
             "| kernel | dispatches | fetch GB | write GB | total GB | algorithmic GB | ratio |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for k, e in sorted(rows.items(), key=lambda kv: -kv[1]["bytes_per_launch"]):
        alg = e.get("algorithmic_bytes")
        lines.append(f"| {k} | {e['dispatches']} | {e['fetch_bytes'] / 1e9:.3f} | "
                     f"{e['write_bytes'] / 1e9:.3f} | {e['bytes_per_launch'] / 1e9:.3f} | "
                     + (f"{alg / 1e9:.3f} | {e['traffic_over_algorithmic']:.2f} |" if alg else "| |"))
    with open(a.summary, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
