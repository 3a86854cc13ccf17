"""The oracle's pins, run again against its AddressSanitizer + UndefinedBehaviorSanitizer
build (oracle/build.py, sanitize=True), in a child interpreter that preloads the
sanitizer runtime.  Any report (an out-of-bounds access, a use after free, signed
overflow, a bad shift, ...) aborts the child and fails this test.  CPU only.
"""
import glob
import os
import subprocess
import sys

from oracle import build as oracle_build

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = oracle_build.build(sanitize=True, out=str(tmp_path / "liboracle_san.so"))
    files = sorted(f for f in glob.glob(os.path.join(TESTS, "test_oracle_*.py"))
                   if not f.endswith(("test_oracle_mutants.py", "test_oracle_sanitized.py")))
    assert len(files) >= 8
    env = dict(os.environ, GS_ORACLE_LIB=lib, LD_PRELOAD=oracle_build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    # the full-size workload checks (marked slow) are left out: their arithmetic is the
    # pins' own, and under the sanitizers they would take minutes
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu and not slow", "-p",
                        "no:cacheprovider"] + files,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "Sanitizer" not in r.stderr, tail
    assert " passed" in r.stdout, tail
