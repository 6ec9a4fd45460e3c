"""The rocprofv3 summariser (no GPU): copy calibration, the clock column, and the traffic record
of the one-launch GEMMs summed over their two launches; the source digest ignores comments and
profiling-only blocks."""
import csv
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from backward_token_expert_amd import rocprof_summary as R  # noqa: E402

FUSED = "void lrm::(anonymous namespace)::gemm_fused<Tile<4, 3, 4, true>, Tile<4, 3, 4, false>, 4, 2, {}>(x)"
COPY = "__amd_rocclr_copyBuffer"


def _pass(root, name, rows):
    d = os.path.join(root, name)
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for kernel, counter, value, dur in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value,
                        "Start_Timestamp": 1000, "End_Timestamp": 1000 + dur})


def test_two_launches_of_the_fused_gemm_are_summed(tmp_path):
    root = str(tmp_path)
    copy_bytes = 1 << 30
    # the copy reads FETCH_SIZE at half its bytes (128-byte requests counted as 64) and WRITE_SIZE
    # at its bytes: scales 2 and 1
    _pass(root, "p1", [(FUSED.format(0), "GRBM_GUI_ACTIVE", 8 * 1_000_000, 1_000_000),
                       (FUSED.format(0), "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 700_000, 1_000_000),
                       (FUSED.format(1), "GRBM_GUI_ACTIVE", 8 * 2_000, 2_000),
                       (FUSED.format(1), "SQ_VALU_MFMA_BUSY_CYCLES", 0, 2_000)])
    _pass(root, "p2", [(COPY, "FETCH_SIZE", copy_bytes // 2 // 1024, 100),
                       (FUSED.format(0), "FETCH_SIZE", 1000, 100),
                       (FUSED.format(1), "FETCH_SIZE", 10, 100)])
    _pass(root, "p3", [(COPY, "WRITE_SIZE", copy_bytes // 1024, 100),
                       (FUSED.format(0), "WRITE_SIZE", 500, 100),
                       (FUSED.format(1), "WRITE_SIZE", 5, 100)])
    text, rec = R.counters_report(root, copy_bytes, "w")
    assert abs(rec["fetch_scale"] - 2.0) < 1e-9 and abs(rec["write_scale"] - 1.0) < 1e-9
    k = rec["kernels"]["lrm_grouped_dw_dx"]
    assert len(k["kernels"]) == 2
    assert k["fetch_bytes"] == (1000 + 10) * 1024 * 2
    assert k["write_bytes"] == (500 + 5) * 1024
    assert k["traffic_bytes"] == k["fetch_bytes"] + k["write_bytes"]
    # clock and MFMA busy of the launch that ran the product: 8e6 / 8 cycles in 1 ms = 1000 MHz
    assert k["kernel"].endswith(", 2, 0>")
    assert abs(k["clock_mhz"] - 1000.0) < 1e-6 and abs(k["mfma_busy_pct"] - 70.0) < 1e-6
    assert k["source_sha256"] == R.source_digest("lrm_grouped_dw_dx")
    assert "| 1000 |" in text  # the clock column


def test_digest_ignores_comments_and_profiling_blocks():
    code = "int a; // note\n/* block */ int b;\n"
    prof = "int a;\n#ifdef LRM_TIMELINE\nint t;\n#if X\nint u;\n#endif\n#endif\nint b;\n"
    assert R._code_only(code) == R._code_only("int a; int b;") == R._code_only(prof)
    assert R._code_only("int a;\n#ifdef OTHER\nint t;\n#endif\n") != R._code_only("int a;")
