"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: its C
source built with both (any report aborts the process) and the oracle pins
run on that build in a child process that preloads the sanitizer runtimes.
ThreadSanitizer is not run: the OpenMP runtime (libgomp) is not built with
it, so every parallel region would report its own synchronisation.  The
oracle's OpenMP loops write disjoint rows; its bits not depending on the
thread count is pinned instead (tests/pins.py)."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.slow
def test_oracle_pins_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    oracle.build(force=True, sanitized=True)
    env = dict(os.environ, MSA_ORACLE_SANITIZED="1", LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    code = ("import sys, oracle, pytest; "
            "rc = pytest.main(['-x', '-q', '-p', 'no:cacheprovider', 'tests/test_oracle_pins.py']); "
            "print('ORACLE_LIB', oracle.loaded_path()); sys.exit(rc)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ORACLE_LIB " + os.path.join(ROOT, "oracle", "liboracle_san.so") in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
