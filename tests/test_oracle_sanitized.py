"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle pins run again in a child process that loads a sanitizer build of
kvarn_oracle.c (host code only, gcc), so an out-of-bounds access, a use of
uninitialised stack through a bad index or undefined integer arithmetic in
the checker fails the suite instead of silently shaping its answers."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from oracle import build as obuild
    obuild.build(sanitize=True)
    env = dict(os.environ)
    env.update({"KVARN_ORACLE_SANITIZED": "1", "LD_PRELOAD": f"{asan}:{ubsan}",
                # the Python interpreter itself is not instrumented: report only
                # what the oracle does, stop at the first error
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    which = subprocess.run([sys.executable, "-c", "import oracle; print(oracle._load()._name)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert which.returncode == 0 and which.stdout.strip().endswith("libkvarn_oracle_san.so"), which
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr, tail
    assert "runtime error" not in r.stderr, tail
