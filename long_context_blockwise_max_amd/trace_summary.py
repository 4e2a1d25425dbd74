"""Kernel-trace summary of one rocprofv3 run as a markdown table.

    rocprofv3 --kernel-trace --stats -d <dir> -o run -- python3 bench.py ...
    python -m long_context_blockwise_max_amd.trace_summary --db <dir>/run_results.db \\
        --title "Kernel trace, 128k workload" --summary profiles/kernel_trace_128k.md \\
        --command "<the lines above>" [--note "<what one step runs>"]

The table is the `top_kernels` view of the run's rocpd database: calls, total and
average duration per kernel (microseconds) and its share of all kernel time.
With --bench-json (the JSON line the profiled benchmark printed) the summary
also carries that line and checks it against the trace: the roofline fraction
recomputed from the traced average of the dominant kernel, beside the one the
benchmark measured with its own events in the same run.
"""
from __future__ import annotations

import argparse
import json
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


def bench_check(kernels, bench_json, prefix):
    """Lines tying the trace to the benchmark line of the same run."""
    with open(bench_json) as fh:
        line = [l for l in fh.read().splitlines() if l.startswith("{")][-1]
    b = json.loads(line)
    roof = b["roofline"]
    match = [k for k in kernels if prefix in k[0].split("(")[0]]
    out = ["", "The benchmark line this profiled run printed:", "", "```", line, "```", ""]
    if not match:
        return out + [f"(no kernel named {prefix}... in the trace)"]
    name, calls, total, avg, _ = match[0]
    flop = b["phase1"]["algorithmic_flop"]
    frac_trace = flop / (avg * 1e-6) / (roof["peak"] * 1e12)
    out += ["Cross-check of the dominant kernel in this one run:", "",
            f"- traced average of `{name.split('(')[0]}` over {calls} launches (warm-up "
            f"included): {avg / 1e3:.3f} ms; the benchmark's own events on the launch stream: "
            f"{roof['launch_ms']:.3f} ms over {b['steps']} timed steps",
            f"- roofline fraction from the trace: {flop / 1e12:.3f} TFLOP / {avg / 1e3:.3f} ms / "
            f"{roof['peak']:.0f} TFLOP/s = {frac_trace:.4f}; the benchmark reports "
            f"{roof['frac']:.4f}",
            f"- the benchmark's whole step took {b['ms_per_step']:.3f} ms by its wall clock, "
            f"{'at least' if b['ms_per_step'] >= avg / 1e3 else 'LESS than'} the traced "
            f"kernel average"]
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--db", required=True)
    ap.add_argument("--title", required=True)
    ap.add_argument("--summary", required=True)
    ap.add_argument("--command", default="")
    ap.add_argument("--note", default="")
    ap.add_argument("--bench-json", default=None,
                    help="file holding the JSON line the profiled benchmark printed")
    ap.add_argument("--kernel", default="phase1_kernel<128, false",
                    help="name prefix of the dominant kernel in the trace")
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
    if a.bench_json:
        lines += bench_check(top_kernels(a.db), a.bench_json, a.kernel)
    with open(a.summary, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
