"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two host programs are built with both sanitizers, failing on the first report:

* the build-time table generator (gen_tables.cpp), in its quick mode (a
  smaller brute-force self-check; the printed tables must equal the ones the
  build generated with the full check);
* libhlwq with its host code instrumented (device code is compiled as usual
  and never launched), driven by the plain C client tests/c_abi_check.c, which
  exercises the host entry points and the argument validation of every device
  entry point.
"""
import os
import shutil
import subprocess

import pytest

from weight_quantization_amd import build as wqb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


def _env(**extra):
    env = dict(os.environ)
    # the HIP runtime keeps allocations for the process lifetime; leaks are not
    # what this checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.update(extra)
    return env


def test_table_generator_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "gen_tables_asan")
    subprocess.run([gxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(wqb.CSRC, "gen_tables.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=_env(HLWQ_GEN_QUICK="1"))
    assert r.returncode == 0, r.stderr[-4000:]
    assert "#define HLWQ_CENTROIDS_5" in r.stdout
    built = os.path.join(wqb.BUILD, "hlwq_tables.inc")
    if os.path.exists(built):
        assert r.stdout == open(built).read()


def test_abi_validation_under_sanitizers(tmp_path):
    if not os.path.exists(CLANG):
        pytest.skip("no ROCm clang")
    if not os.path.exists(os.path.join(wqb.BUILD, "hlwq_tables.inc")):
        wqb.generate_tables()
    lib = str(tmp_path / "libhlwq_asan.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-g"]
    r = subprocess.run([wqb._hipcc(), *wqb.HIPCC_FLAGS, *san, "-I", wqb.INCLUDE, "-I", wqb.BUILD,
                        os.path.join(wqb.CSRC, "hlwq.hip"), "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = str(tmp_path / "c_abi_asan")
    subprocess.run([CLANG, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
                    "-L", str(tmp_path), "-lhlwq_asan", "-Wl,-rpath," + str(tmp_path), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=_env())
    assert r.returncode == 0, r.stderr[-4000:]
    assert "c abi ok" in r.stdout
