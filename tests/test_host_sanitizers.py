"""The library's host C++ (chunk-table builder and chunk-table producer, which
need no GPU) built with g++ under AddressSanitizer + UndefinedBehaviorSanitizer
and, separately, ThreadSanitizer (the producer fingerprints requests on host
threads), and run over random tables, planted table defects, CDC streams,
xxHash64 at every length up to 300, and registry batches on 1 and 8 threads
(tests/host_sanitize/driver.cpp).  Any sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_position_independent_amd", "csrc")
SOURCES = [os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp"), os.path.join(CSRC, "irm_table.cpp"),
           os.path.join(CSRC, "irm_producer.cpp")]


def _build_and_run(tmp_path, name, san_flags, env_extra):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / name)
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *san_flags, f"-I{os.path.join(ROOT, 'include')}",
           f"-I{CSRC}", *SOURCES, "-o", exe, "-pthread"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    env = dict(os.environ, **env_extra)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "host checks ok" in run.stdout
    assert "Sanitizer" not in run.stderr, run.stderr
    return run.stdout


def test_host_code_under_address_and_undefined_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "driver_asan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                         {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:halt_on_error=1",
                          "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    assert "table rows" in out


def test_host_code_under_thread_sanitizer(tmp_path):
    out = _build_and_run(tmp_path, "driver_tsan", ["-fsanitize=thread"], {"TSAN_OPTIONS": "halt_on_error=1"})
    assert "producer entries" in out
