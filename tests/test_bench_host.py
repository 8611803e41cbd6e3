"""Host-side checks of bench.py's contract (no GPU)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_bank_workloads():
    # bf16 in + 80 B of codes + 2 B of norm per 128-block (Q5); the tail block
    # of a 704-wide row is stored whole
    assert bench.algorithmic_bytes([(256, 1024, 2048), (256, 2048, 512)], 5) == 2_126_512_128
    assert bench.algorithmic_bytes([(128, 1408, 2816), (128, 2816, 704)], 5) == 2_024_996_864
    assert bench.algorithmic_bytes([(1, 64, 256)], 5) == 43_264
    assert bench.algorithmic_bytes([(1, 5120, 5120)], 3) == 52_428_800 + 10_240_000
    # TQ3: 48 B of codes and a 4-byte fp32 norm per group of 128
    assert bench.algorithmic_bytes([(256, 1024, 2048), (256, 2048, 512)], 3, 4) == 1_937_768_448


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


def test_committed_counters_are_read_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    # traffic and VALU counts come from the committed rocprofv3 summaries, and
    # only while the kernel source they were taken on is unchanged
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "hbm_traffic_x_q5.txt").write_text(
        "# comment: ignored\nkernel_source_sha256_16: %s\nquantize_bytes_per_launch: 100\n"
        "dequantize_bytes_per_launch: 200\n" % bench.kernel_source_hash())
    (prof / "counters_x_q5.md").write_text(
        "# Instruction counters\n\nCommands (MI355X, one GPU):\n\nkernel_source_sha256_16: %s\n"
        "valu_ops_per_value_quantize: 15.06\nvalu_ops_per_value_dequantize: 8.97\n" % bench.kernel_source_hash())
    (prof / "counters_y_q5.md").write_text(
        "kernel_source_sha256_16: 0000000000000000\nvalu_ops_per_value_quantize: 1\nvalu_ops_per_value_dequantize: 2\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: open(prof / "counters_x_q5.md").read().split(
        "kernel_source_sha256_16: ")[1][:16])
    assert bench.stored_traffic("x", 5) == {"quantize_bytes_per_launch": 100.0, "dequantize_bytes_per_launch": 200.0}
    v = bench.stored_valu("x", 5)
    assert v["quantize"] == 15.06 and v["dequantize"] == 8.97
    assert bench.stored_valu("y", 5) is None          # taken on other source
    assert bench.stored_valu("z", 5) is None          # no summary
    assert bench.stored_traffic("z", 5) is None



def test_valu_rate_against_the_issue_peak():
    # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
    assert abs(bench.VALU_PEAK_TOPS - 39.3216) < 1e-9
    # 16 ops per value over 2.4576e9 values in 1 ms: 39.3216 T lane-ops/s, the peak
    r = bench.valu_rate(16.0, 2_457_600_000, 1.0)
    assert r["unit"] == "T VALU lane-ops/s" and abs(r["achieved"] - 39.32) < 0.01 and abs(r["frac"] - 1.0) < 1e-4
    r = bench.valu_rate(15.06, 805_306_368, 0.378)
    assert abs(r["achieved"] - 15.06 * 805_306_368 / 0.378e-3 / 1e12) < 0.01
    assert bench.valu_rate(None, 1, 1.0) is None


def test_roofline_is_the_more_used_of_memory_and_valu():
    valu_low = {"achieved": 18.7, "peak": 39.32, "unit": "T VALU lane-ops/s", "frac": 0.476}
    r = bench.roofline_of("dequantize", 5536.7, 5540.2, valu_low)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["frac"] == round(5536.7 / 8000, 4)
    assert r["valu"] == valu_low and r["frac_of_ceiling"] == round(5536.7 / 5540.2, 4)
    valu_high = {"achieved": 34.2, "peak": 39.32, "unit": "T VALU lane-ops/s", "frac": 0.87}
    r = bench.roofline_of("kv quantize", 4920.0, 5900.0, valu_high)
    assert r["bound"] == "alu" and r["frac"] == 0.87 and r["unit"] == "T VALU lane-ops/s"
    assert r["hbm"]["achieved"] == 4920.0 and r["hbm"]["frac"] == round(4920.0 / 8000, 4)
    assert bench.roofline_of("x", 4000.0, 5000.0, None)["bound"] == "hbm"
