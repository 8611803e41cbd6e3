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
