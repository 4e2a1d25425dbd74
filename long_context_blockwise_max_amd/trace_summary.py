"""Kernel-trace summary of one rocprofv3 run as a markdown table.

    rocprofv3 --kernel-trace --stats -d <dir> -o run -- python3 bench.py ...
    python -m long_context_blockwise_max_amd.trace_summary --db <dir>/run_results.db \\
        --title "Kernel trace, 128k workload" --summary profiles/kernel_trace_128k.md \\
        --command "<the lines above>" [--note "<what one step runs>"]

The table is the `top_kernels` view of the run's rocpd database: calls, total and
average duration per kernel (microseconds) and its share of all kernel time.
"""
from __future__ import annotations

import argparse
import sqlite3


def top_kernels(db: str):
    """[(name, calls, total_us, average_us, percent)] from the rocpd `top_kernels` view
    (its durations are in microseconds)."""
    con = sqlite3.connect(db)
    try:
        cols = [r[1] for r in con.execute("pragma table_info(top_kernels)")]
        rows = list(con.execute("select * from top_kernels"))
    finally:
        con.close()
    ix = {c.lower(): i for i, c in enumerate(cols)}
    out = []
    for r in rows:
        name = r[ix["name"]]
        calls = int(r[ix["total_calls"]])
        total = float(r[ix["total_duration"]])
        avg = float(r[ix["average"]])
        pct = float(r[ix["percentage"]])
        out.append((name, calls, total, avg, pct))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--db", required=True)
    ap.add_argument("--title", required=True)
    ap.add_argument("--summary", required=True)
    ap.add_argument("--command", default="")
    ap.add_argument("--note", default="")
    a = ap.parse_args(argv)
    lines = [f"# {a.title}", ""]
    if a.note:
        lines += [a.note, ""]
    lines += ["Command:", "", "```", a.command.strip(), "```", "",
              "Summary (the `top_kernels` view of the run's rocpd database; durations in "
              "microseconds):", "",
              "| kernel | calls | total us | average us | % |", "|---|---:|---:|---:|---:|"]
    for name, calls, total, avg, pct in top_kernels(a.db):
        short = name.split("(")[0]          # the argument list adds nothing
        lines.append(f"| `{short}` | {calls} | {total:.1f} | {avg:.1f} | {pct:.2f} |")
    with open(a.summary, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
