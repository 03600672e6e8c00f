"""The host-only library (planner, arena planner, blob parser, pass metadata
builder and checker) built with -fsanitize=address,undefined and driven by
tests/host_sanitized_driver.py in a child process with the AddressSanitizer
runtime preloaded; any report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p) else None


def test_host_library_under_asan_and_ubsan(tmp_path):
    from encoder_scoring_amd import build
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no libasan in this toolchain")
    lib = build.build_host(extra_flags=["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                        "-fno-omit-frame-pointer", "-O1"],
                           out=str(tmp_path / "libencscore_host_asan.so"))
    env = dict(os.environ, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "host_sanitized_driver.py"), lib],
                       capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "planner / metadata calls ok" in out
