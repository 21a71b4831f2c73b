"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
every CPU pin of the oracle (tests/test_oracle_*.py) runs again, in a child
process, against liboracle_san.so (the same source built with
-fsanitize=address,undefined, any finding fatal).  An out-of-bounds access,
use after free, signed overflow, misaligned or out-of-range shift anywhere in
the oracle fails this test."""
import glob
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    path = subprocess.check_output(["gcc", "-print-file-name=%s" % name], text=True).strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(900)
def test_oracle_pins_under_sanitizers():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    oracle.build(force=True, sanitized=True)
    files = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    assert files
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env[oracle.SANITIZED_ENV] = "1"
    # Python's own allocations are not the subject: no leak report at exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"] + files,
                       cwd=ROOT, env=env, capture_output=True, text=True)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
