"""The oracle's pins, re-run against an AddressSanitizer + UndefinedBehaviorSanitizer
build of oracle/path_oracle.c (ORACLE_SANITIZE=1, sanitizer runtimes preloaded
into a child Python process): any out-of-bounds access, use after free or
undefined behaviour in the C oracle aborts the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    try:
        path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not available")
    env = dict(os.environ, ORACLE_SANITIZE="1", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", LD_PRELOAD=f"{asan}:{ubsan}")
    env.pop("PYTEST_ADDOPTS", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_project.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert os.path.exists(os.path.join(ROOT, "oracle", "_build", "liboracle_asan_ubsan.so"))
