"""Host logic of the counter summaries (no GPU): kernel-name mapping, the
comment-insensitive source digest and the copy calibration."""
import csv

from lm_head_vocab_amd import profiling as P


def test_trace_name_mapping():
    assert P.trace_name("void specloss::k_gemm<unsigned short, float, 1, false>(specloss::GemmLaunch)") == "gemm_dW"
    assert P.trace_name("void specloss::k_gemm<unsigned short, float, 0, false>(specloss::GemmLaunch)") == "gemm_dh"
    assert P.trace_name("void specloss::k_gemm<unsigned short, float, 0, false, 4, false>(specloss::GemmLaunch)") == "gemm_dh"
    assert P.trace_name("void specloss::k_gemm<unsigned short, float, 0, false, 4, true>(specloss::GemmLaunch)") == "gemm_dh_dzt"
    assert P.trace_name("void specloss::k_gemm<unsigned short, float, 1, false, 4, false>(specloss::GemmLaunch)") == "gemm_dW"
    assert P.trace_name("void specloss::k_stats<unsigned short, true>(specloss::StatsLaunch)") == "stats_p"
    assert P.trace_name("void specloss::k_stats<unsigned short, false>(specloss::StatsLaunch)") == "stats_q"
    assert P.trace_name("void specloss::k_stats<unsigned short, false, 4, true>(specloss::StatsLaunch)") == "stats_q"
    assert P.trace_name("void specloss::k_stats<unsigned short, true, 4, true>(specloss::StatsLaunch)") == "stats_p"
    assert P.trace_name("void specloss::k_div_raw<7u>(specloss::DivRawLaunch)") == "div_raw"
    assert P.trace_name("void specloss::k_dz_raw<unsigned short, true>(specloss::DzRawLaunch)") == "dz_raw"
    assert P.trace_name("void specloss::k_div<unsigned short, 2, 7u>(specloss::DivLaunch)") == "div"
    assert P.trace_name("void specloss::k_stats_stage<unsigned short>(specloss::StatsStageLaunch)") == "stats_stage"
    assert P.trace_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_code_only_ignores_comments_and_layout():
    a = "int x = 1; // one\n/* block\n comment */ int y = 2;\n"
    b = "int x = 1;\n\n   int y = 2;   // two\n"
    assert P._code_only(a) == P._code_only(b) == "int x = 1; int y = 2;"
    assert P._code_only("int x = 1;") != P._code_only("int x = 2;")


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerows(rows)


def test_summarize_scales_by_the_copy(tmp_path):
    copy, gemm = "__amd_rocclr_copyBuffer", "void specloss::k_gemm<unsigned short, float, 1, false>(x)"
    # the copy of 1 MiB reads as 512 KiB fetched and 1024 KiB written
    _write(tmp_path / "f.csv", [
        {"Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 512.0},
        {"Kernel_Name": gemm, "Counter_Name": "FETCH_SIZE", "Counter_Value": 100.0},
        {"Kernel_Name": gemm, "Counter_Name": "FETCH_SIZE", "Counter_Value": 300.0}])
    _write(tmp_path / "w.csv", [
        {"Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1024.0},
        {"Kernel_Name": gemm, "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0}])
    s = P.summarize(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1 << 20)
    assert s["factor_fetch"] == 2.0 and s["factor_write"] == 1.0
    k = s["kernels"]["gemm_dW"]
    assert k["dispatches"] == 2
    assert k["fetch_bytes"] == 200.0 * 1024 * 2.0      # mean of the dispatches, scaled
    assert k["write_bytes"] == 10.0 * 1024 * 1.0
    assert s["source_digest"] == P.source_digest()


def test_summarize_adds_kernels_of_one_launch(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    main = "void specloss::k_gemm<unsigned short, float, 1, false, 256>(x)"
    tail = "void specloss::k_gemm<unsigned short, float, 1, false, 128>(x)"
    rows = [{"Kernel_Name": copy, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1024.0}]
    for _ in range(3):
        rows.append({"Kernel_Name": main, "Counter_Name": "FETCH_SIZE", "Counter_Value": 90.0})
        rows.append({"Kernel_Name": tail, "Counter_Name": "FETCH_SIZE", "Counter_Value": 10.0})
    _write(tmp_path / "f.csv", rows)
    _write(tmp_path / "w.csv", [{"Kernel_Name": copy, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1024.0}])
    s = P.summarize(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1 << 20)
    k = s["kernels"]["gemm_dW"]
    assert k["dispatches"] == 3 and k["kernels"] == 2
    assert k["fetch_bytes"] == 100.0 * 1024      # main + tail per launch, factor 1



def test_markdown_lists_kernels_traffic_and_bench(tmp_path):
    with open(tmp_path / "stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": "void specloss::k_gemm<unsigned short, float, 1, false>(specloss::GemmLaunch)",
                    "Calls": 4, "TotalDurationNs": 4e6, "AverageNs": 1e6, "Percentage": 100.0})
    traffic = {"copy_kernel": "__amd_rocclr_copyBuffer", "copy_bytes": 1 << 30, "factor_fetch": 2.0,
               "factor_write": 1.0, "source_digest": "abc",
               "kernels": {"gemm_dW": {"fetch_bytes": 2e9, "write_bytes": 1e9, "bytes_per_launch": 3e9}}}
    bench = {"value": 1000.0, "unit": "tokens/s", "ms_per_step": 4.0,
             "roofline": {"kernel": "gemm_dW", "avg_launch_ms": 1.0, "achieved": 100.0,
                          "unit": "TFLOP/s", "frac": 0.04}}
    md = P.markdown(str(tmp_path / "stats.csv"), traffic, "ce_bf16_8b", bench)
    assert "| `void k_gemm<unsigned short, float, 1, false>(GemmLaunch)` | 4 | 1.0000 |" in md
    assert "| gemm_dW | 2.000 | 1.000 | 3.000 |" in md
    assert "--workload ce_bf16_8b" in md and "`gemm_dW` 1.0000 ms per launch" in md


def test_single_call_average_takes_the_first_dispatches(tmp_path):
    """bench.py runs the single call's steps first: the kernel's first
    TRACE_STEPS x launches-per-step dispatches are that call's."""
    path = tmp_path / "run_kernel_trace.csv"
    gemm = "void specloss::k_gemm<unsigned short, float, 1, false, 4>(specloss::GemmLaunch)"
    other = "void specloss::k_dz_raw<unsigned short, false>(specloss::DzRawLaunch)"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for i in range(P.TRACE_STEPS * 2 + 3):  # two launches per step, then three longer ones
            dur = 1_000_000 if i < P.TRACE_STEPS * 2 else 9_000_000
            w.writerow({"Kernel_Name": gemm, "Start_Timestamp": t, "End_Timestamp": t + dur})
            w.writerow({"Kernel_Name": other, "Start_Timestamp": t, "End_Timestamp": t + 5})
            t += dur
    assert P.single_call_avg_ms(str(path), "gemm_dW", 2.0) == 1.0
    assert P.single_call_avg_ms(str(path), "gemm_dW", 10.0) is None
