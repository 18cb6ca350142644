"""Host sanitizer builds: the library's host code (format builders, window
split, reordering, status) and the C oracle, each built with AddressSanitizer
and UndefinedBehaviorSanitizer and driven over random and malformed inputs by
its own driver under tests/sanitize/.  Any invalid access, leak or undefined
behaviour ends the driver with a non-zero status.  CPU only (g++/gcc)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "window_spmm_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(cmd, exe, tmp_path):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout
    r = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       env=ENV, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-4000:]


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_library_host_code_under_asan_ubsan(tmp_path):
    exe = tmp_path / "host_driver"
    srcs = [os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")] + \
        [os.path.join(CSRC, f) for f in ("formats.cpp", "reorder.cpp", "status.cpp")]
    cmd = ["g++", "-std=c++17"] + SAN + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + srcs + \
        ["-o", str(exe)]
    _build_and_run(cmd, exe, tmp_path)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=c11"] + SAN + [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                                      os.path.join(ROOT, "oracle", "spmm_oracle.c"),
                                      "-pthread", "-lm", "-o", str(exe)]
    _build_and_run(cmd, exe, tmp_path)
