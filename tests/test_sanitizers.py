"""CPU sanitizer pass over the oracle: mra_oracle.c built with
AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts) runs the
whole pin suite.  An out-of-bounds access, a use after free or undefined
integer arithmetic anywhere the pins reach fails this test."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mra_oracle.c")


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc has no AddressSanitizer runtime here")
def test_oracle_pins_under_address_and_undefined_sanitizers(tmp_path):
    so = str(tmp_path / "libmra_oracle_san.so")
    flags = [f for f in oracle.CFLAGS if f != "-O2"]
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", *flags, SRC, "-o", so, "-lm"])
    env = dict(os.environ, MRA_ORACLE_LIB=so, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
