"""The host half of libbcg (bcg_host.cpp: sigma schedules, bucket tables,
plans, sample records, area slices) built on its own by g++ with
AddressSanitizer and UndefinedBehaviorSanitizer, and the ``host`` cases of
test_host_lib.py run against that build in a child process: any invalid
access, overflow or undefined operation in the host code ends the child with
a report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bucketed_classifier_free_amd", "csrc")


def _runtime(gxx, name):
    path = subprocess.run([gxx, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_half_clean_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    asan = _runtime(gxx, "libasan.so")
    if asan is None or _runtime(gxx, "libubsan.so") is None:
        pytest.skip("the sanitizer runtimes are not installed")
    so = str(tmp_path / "libbcg_host_san.so")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fPIC", "-shared"]
    subprocess.run([gxx] + flags + ["-I", os.path.join(ROOT, "include"), "-I", CSRC,
                                    os.path.join(CSRC, "bcg_host.cpp"), "-o", so], check=True)
    pre = os.environ.get("LD_PRELOAD", "")
    env = dict(os.environ,
               LD_PRELOAD=asan + (":" + pre if pre else ""),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               BCG_SANITIZED_HOST_LIB=so,
               PYTHONPATH=os.pathsep.join([os.path.join(ROOT, "tests"), ROOT]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "sanitized_host", "-p", "no:cacheprovider",
                        "-m", "host", os.path.join(ROOT, "tests", "test_host_lib.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]
    summary = [ln for ln in r.stdout.splitlines() if " passed" in ln]
    assert summary and "failed" not in summary[-1] and "deselected" in summary[-1], out[-2000:]
