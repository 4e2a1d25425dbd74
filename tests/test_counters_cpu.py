"""Host logic of the counter summary: per-dispatch sums over counter instances,
copy-kernel calibration, and the source-hash gate bench.py applies."""
import csv
import json

from long_context_blockwise_max_amd import source_hash as SH
from long_context_blockwise_max_amd import counters

HEAD = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(HEAD)
        for disp, name, vals in rows:
            for v in vals:          # several instances (e.g. one per L2 channel group)
                w.writerow([disp, disp, "Agent 1", 1, 1, 1, 64, 1, name, 256, 0, 0, 8, 0, 16,
                            counter, v, 0, 1])


def test_summary_scales_by_copy_and_gates_on_source(tmp_path):
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(...)"
    p1 = "void pulsar::phase1_kernel<128, false>(pulsar::P1Args)"
    # copy of 1 MiB reads 1024 KiB reported as 512 + 512; phase1 twice
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(1, copy, [512.0, 512.0]), (2, p1, [1000.0, 1000.0]),
                                             (3, p1, [1500.0, 1500.0])])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(1, copy, [256.0, 256.0]), (2, p1, [100.0]),
                                             (3, p1, [300.0])])
    out, md = tmp_path / "t.json", tmp_path / "t.md"
    counters.main(["--fetch", str(tmp_path / "f.csv"), "--write", str(tmp_path / "w.csv"),
                   "--copy-mib", "1", "--workload", "tiny", "--out", str(out), "--summary", str(md),
                   "--command", "rocprofv3 ..."])
    rec = json.loads(out.read_text())
    e = rec["kernels"]["tiny"]["phase1_kernel"]
    assert e["dispatches"] == 2
    assert e["fetch_bytes"] == 2500 * 1024          # fetch scale 1.0
    assert e["write_bytes"] == 200 * 1024 * 2       # write scale 2.0
    assert rec["source_hash"] == SH.kernel_source_hash()
    assert "phase1_kernel" in md.read_text()


def test_template_forms_are_told_apart():
    assert counters.short_name("void pulsar::phase1_kernel<128, false>(pulsar::P1Args)") == "phase1_kernel"
    assert counters.short_name("void pulsar::phase1_kernel<128, true>(pulsar::P1Args)") == "phase1_kernel_prefix_rows"
    assert counters.short_name("void pulsar::phase2_kernel<64, true>(pulsar::P2Args)") == "phase2_kernel_decode"
    # a third template argument (the wave count) keeps the form
    assert counters.short_name("void pulsar::phase1_kernel<128, false, 12>(pulsar::P1Args)") == "phase1_kernel"
    assert counters.short_name("void pulsar::phase1_kernel<64, true, 8>(pulsar::P1Args)") == "phase1_kernel_prefix_rows"


def test_matrix_summary_per_dispatch_and_over_compute(tmp_path):
    from long_context_blockwise_max_amd import matrix_counters as M
    import workloads as W
    p1 = "void pulsar::phase1_kernel<128, false>(pulsar::P1Args)"
    w = W.WORKLOADS["tiny"]
    alg = M.algorithmic_flops(w, "phase1_kernel")
    mops = alg * 1.25 / 512.0                # 25 % over-compute, split over 2 instances
    path = tmp_path / "m.csv"
    with open(path, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(HEAD)
        for disp in (1, 2):
            for cname, vals in ((M.MOPS, [mops / 2, mops / 2]), (M.BUSY, [300.0, 212.0]),
                                (M.GUI, [8.0])):
                for v in vals:
                    wr.writerow([disp, disp, "Agent 1", 1, 1, 1, 64, 1, p1, 256, 0, 0, 8, 0, 16,
                                 cname, v, 0, 1])
    rows = M.per_kernel(str(path))
    e = rows["phase1_kernel"]
    assert e["dispatches"] == 2
    assert abs(e["mfma_flop"] / alg - 1.25) < 1e-9
    # busy summed over instances; active cycles arrive summed over the 8 XCDs
    assert abs(e["mfma_busy"] - 512.0 / 1024) < 1e-12
    md = tmp_path / "m.md"
    M.main(["--pmc", str(path), "--workload", "tiny", "--summary", str(md)])
    assert "1.250" in md.read_text()


def test_trace_summary_reads_the_top_kernels_view(tmp_path):
    import sqlite3
    from long_context_blockwise_max_amd import trace_summary as T
    db = tmp_path / "r.db"
    con = sqlite3.connect(db)
    con.execute("create table top_kernels (name text, total_calls int, total_duration real, "
                "average real, percentage real)")
    con.execute("insert into top_kernels values ('void pulsar::phase1_kernel<128, false>(pulsar::P1Args)',"
                " 6, 189528.9, 31588.15, 93.78)")
    con.commit()
    con.close()
    rows = T.top_kernels(str(db))
    assert rows == [("void pulsar::phase1_kernel<128, false>(pulsar::P1Args)", 6, 189528.9, 31588.15, 93.78)]
    md = tmp_path / "t.md"
    T.main(["--db", str(db), "--title", "Kernel trace", "--summary", str(md), "--command", "rocprofv3 ..."])
    assert "| `void pulsar::phase1_kernel<128, false>` | 6 | 189528.9 | 31588.2 | 93.78 |" in md.read_text()


def test_code_hash_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* plain */ }\n"
    b = "int f(int x) {\n  // twice x\n  return 2 * x;\n}\n"
    c = "int f(int x) { return 3 * x; }"
    assert SH.code_text(a) == SH.code_text(b)
    assert SH.code_text(a) != SH.code_text(c)
    assert "s_waitcnt vmcnt(0)" in SH.code_text('asm volatile("s_waitcnt vmcnt(0)");  // wait')
