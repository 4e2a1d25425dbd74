"""Matrix-core work per kernel launch from one rocprofv3 counter run.

One `--pmc` pass of the bench command with
    SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
gives, per dispatch, the bf16 MFMA work (the counter counts multiply and add
operations divided by 512), the cycles the matrix cores were busy summed over
every SIMD (32 per 32x32x16 bf16 instruction), and the GPU's active cycles.
GRBM_GUI_ACTIVE arrives as one value summed over the 8 XCDs: an eighth of it
divided by the dispatch's duration is the clock (2.2-2.45 GHz on short
dispatches of this chip).  From them:

    mfma_flop    = 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16
    over-compute = mfma_flop / the launch's algorithmic FLOPs
                   (padding rows, masked diagonal keys, rounded-up tiles)
    mfma_busy    = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 1024 SIMDs)
    clock        = GRBM_GUI_ACTIVE / 8 / duration   (where the run recorded times)

    python -m long_context_blockwise_max_amd.matrix_counters \\
        --pmc <run>/run_counter_collection.csv (or run_results.db) \\
        --workload 128k --summary profiles/mfma_128k.md --command "<the rocprofv3 line>"
"""
from __future__ import annotations

import argparse
import collections
import os
import sys

from .counters import _records, short_name

N_SIMD = 256 * 4
N_XCD = 8
MOPS = "SQ_INSTS_VALU_MFMA_MOPS_BF16"
BUSY = "SQ_VALU_MFMA_BUSY_CYCLES"
GUI = "GRBM_GUI_ACTIVE"


def per_kernel(path: str):
    """{short kernel name: {"dispatches", "mfma_flop", "busy", "gui"}} averaged per dispatch.
    MFMA counters are summed over their instances; the GPU-active count is the
    maximum over its instances (every instance sees the same window)."""
    acc = collections.defaultdict(lambda: {MOPS: 0.0, BUSY: 0.0, GUI: 0.0})
    names = {}
    dur = _durations(path)
    for d, name, cname, value in _records(path):
        d = int(d)
        names[d] = short_name(name)
        if cname in (MOPS, BUSY):
            acc[d][cname] += float(value)
        elif cname == GUI:
            acc[d][GUI] = max(acc[d][GUI], float(value))
    out = {}
    for d in sorted(acc):
        e = out.setdefault(names[d], {"dispatches": 0, "mfma_flop": 0.0, "busy": 0.0, "gui": 0.0,
                                      "seconds": 0.0, "timed": 0})
        e["dispatches"] += 1
        e["mfma_flop"] += acc[d][MOPS] * 512.0
        e["busy"] += acc[d][BUSY]
        e["gui"] += acc[d][GUI] / N_XCD
        if dur.get(d, 0.0) > 0:
            e["seconds"] += dur[d]
            e["timed"] += 1
    for e in out.values():
        n = e["dispatches"]
        e["mfma_flop"] /= n
        e["busy"] /= n
        e["gui"] /= n
        e["mfma_busy"] = e["busy"] / (e["gui"] * N_SIMD) if e["gui"] > 0 else None
        e["clock_ghz"] = None
        if e["timed"] == n:
            e["seconds"] /= n
            e["clock_ghz"] = e["gui"] / e["seconds"] / 1e9
    return out


def _durations(path: str):
    """{dispatch id: seconds} from the start and end stamps of a counter collection
    (nanoseconds), where the run recorded them."""
    out = {}
    if path.endswith(".db"):
        import sqlite3
        con = sqlite3.connect(path)
        try:
            for d, s, e in con.execute("select dispatch_id, min(start), max(end) "
                                       "from counters_collection group by dispatch_id"):
                if s is not None and e is not None and e > s:
                    out[int(d)] = (e - s) * 1e-9
        finally:
            con.close()
        return out
    import csv
    with open(path) as fh:
        for r in csv.DictReader(fh):
            s, e = float(r.get("Start_Timestamp") or 0), float(r.get("End_Timestamp") or 0)
            if e > s:
                out[int(r["Dispatch_Id"])] = (e - s) * 1e-9
    return out


def algorithmic_flops(w, kernel):
    """FLOPs the launch must compute: Phase 1 over block-row queries, Phase 2 over
    the query rows, the prefix rows over the last block's prefix list."""
    from . import costs as C
    k = w.k_eff
    if kernel == "phase1_kernel":
        return C.phase1_flops_rows(w.n_blocks, w.block_size, w.sink_size, w.chunk_size, k,
                                   w.n_q_heads, w.head_dim)
    if kernel == "phase2_kernel" or kernel == "phase2_kernel_decode":
        return C.phase2_flops(w.batch, w.q_len, w.context_len, w.n_q_heads, w.head_dim)
    if kernel == "phase1_kernel_prefix_rows" and w.n_blocks > 1:
        n = w.sink_size + w.chunk_size * k * (w.n_blocks - 1)
        return C.prefix_rows_flops(n, w.n_q_heads, w.head_dim)
    return None


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--pmc", required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--summary", required=True)
    ap.add_argument("--command", default="")
    a = ap.parse_args(argv)

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import workloads as W

    w = W.WORKLOADS[a.workload]
    rows = per_kernel(a.pmc)
    lines = [f"# Matrix-core work per launch, {a.workload} workload", "",
             "Command:", "", "```", a.command.strip(), "```", "",
             "mfma GFLOP = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16; over-compute = that / the "
             "algorithmic FLOPs; busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 "
             "SIMDs); clock = GRBM_GUI_ACTIVE / 8 / the dispatch's duration under the profiler.",
             "",
             "| kernel | dispatches | mfma GFLOP | algorithmic GFLOP | over-compute | MFMA busy | clock GHz |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for k, e in sorted(rows.items(), key=lambda kv: -kv[1]["mfma_flop"]):
        if e["mfma_flop"] <= 0:
            continue
        alg = algorithmic_flops(w, k)
        busy = e["mfma_busy"]
        lines.append(f"| {k} | {e['dispatches']} | {e['mfma_flop'] / 1e9:.1f} | "
                     + (f"{alg / 1e9:.1f} | {e['mfma_flop'] / alg:.3f} |" if alg else "| |")
                     + (f" {100 * busy:.1f} % |" if busy is not None else " |")
                     + (f" {e['clock_ghz']:.2f} |" if e["clock_ghz"] else " |"))
    with open(a.summary, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
