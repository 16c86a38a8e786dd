"""The oracle built under AddressSanitizer and UBSan (CPU only): every exported
oracle function on small problems in every storage type and masking mode,
with exact-size buffers (oracle/sanitize_main.c), must run clean, leaks
included.  A read or write past a buffer, or undefined behaviour, fails the
test with the sanitizer's report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = tmp_path / "oracle_sanitized"
    build = subprocess.run(
        [gcc, "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "attn_oracle.c"),
         os.path.join(ROOT, "oracle", "sanitize_main.c"), "-lm", "-o", str(exe)],
        capture_output=True, text=True, timeout=300)
    if build.returncode != 0 and "sanitize" in build.stderr and "unrecognized" in build.stderr:
        pytest.skip("this gcc has no sanitizer runtime")
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert run.stdout.startswith("ok:"), run.stdout
