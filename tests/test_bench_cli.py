"""bench.py's command line on the CPU: runs on more than one GPU are refused
with a message before any GPU work (the R ranks are virtual ranks in one
GPU), and the profile summarisers turn small counter files into summaries."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout


def test_stats_summary_from_a_small_csv(tmp_path):
    csv = tmp_path / "k_stats.csv"
    csv.write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void moonep::k_gemm<2>(moonep::GemmArgs)",2,34000000,17000000,60.0,16900000,17100000,1\n'
        '"void moonep::k_dispatch<4>(int)",2,3200000,1600000,40.0,1590000,1610000,1\n')
    out = tmp_path / "summary.md"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-stats",
                        str(csv), "cmd", str(out)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    text = out.read_text()
    assert "| k_gemm<2> | 2 | 17000.0 |" in text
    assert "| k_dispatch | 2 | 1600.0 |" in text


def test_source_digest_ignores_comments_only():
    sys.path.insert(0, ROOT)
    import bench
    a = "int f(int x) {  // one\n  return x + 1; /* two\n lines */ }\n"
    b = "int f(int x) {\n  return x + 1; }  // changed comment\n"
    c = "int f(int x) {\n  return x + 2; }\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_vendor_kernel_rows_are_named_by_tile():
    sys.path.insert(0, ROOT)
    import bench
    name = "Cijk_Ailk_Bljk_BBS_BH_Bias_HA_S_SAV_UserArgs_MT256x256x64_MI16x16x1_SN_LDSB1"
    assert bench._short_kernel(name) == "hipBLASLt Cijk MT256x256x64 MI16x16x1"
    assert bench._short_kernel("void moonep::k_gemm<2>(moonep::GemmArgs)") == "k_gemm<2>"
    assert bench._short_kernel("void moonep::k_gemm<0, 4>(moonep::GemmArgs)") == "k_gemm<0>"
    assert bench._short_kernel("void moonep::k_gemm<2, 1>(moonep::GemmArgs)") == "k_gemm<2>c1"
    assert bench._short_kernel("void moonep::k_sched<0>(moonep::SchedArgs)") == "k_sched<0>"
    assert bench._short_kernel("void moonep::k_route<true>(moonep::PlanArgs)") == "k_route"
