"""The oracle's pins again, against a build of oracle.c with AddressSanitizer
and UndefinedBehaviorSanitizer (gcc, host code only): any out-of-bounds
access, use of freed memory or undefined operation in the oracle fails it."""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    try:
        path = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                              capture_output=True, text=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _asan_runtime() is None,
                    reason="gcc with the AddressSanitizer runtime is not installed")
def test_oracle_pins_under_address_and_undefined_sanitizers(tmp_path):
    so = str(tmp_path / "liboracle_asan.so")
    subprocess.run(["gcc", *oracle.CFLAGS, "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-o", so, oracle.SRC, "-lm"], check=True)
    env = dict(os.environ)
    env.update({
        "ORACLE_LIB": so,
        "LD_PRELOAD": _asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in tail and "runtime error" not in tail
