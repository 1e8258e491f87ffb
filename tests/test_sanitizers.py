"""CPU sanitizer builds (AddressSanitizer + UndefinedBehaviorSanitizer):

* the C oracle, driven by tests/native/oracle_sanitize.c;
* the library's host-side validation layer (size checks, workspace layout,
  device-content precondition checks; csrc/gdn_validate.cpp, which has no
  HIP dependency), driven by tests/native/validate_sanitize.cpp.

Each is compiled with gcc/g++ into a temporary directory and must run clean:
any out-of-bounds access, use after free, leak, signed overflow or other
undefined behaviour aborts the driver with a report.  Host code only: no GPU
code is built with a sanitizer.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "hybrid_linear_attention_gdn_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    _run(["gcc", "-std=c11", "-fopenmp", *SAN, "-o", exe, os.path.join(NATIVE, "oracle_sanitize.c"),
          os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm"], str(tmp_path))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_validation_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "validate_sanitize")
    _run(["g++", "-std=c++17", *SAN, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-o", exe,
          os.path.join(NATIVE, "validate_sanitize.cpp"), os.path.join(CSRC, "gdn_validate.cpp")], str(tmp_path))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout + r.stderr
