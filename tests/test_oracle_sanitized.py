"""The oracle's pin suite once more, against a build of the oracle with
AddressSanitizer and UndefinedBehaviorSanitizer (host code only): the oracle
sizes several heap arrays by arithmetic (packed rows, K-major block-row
lists), and an out-of-bounds access or undefined operation there must show up
as a failure here rather than as a silently wrong expected value."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mxfp4_oracle.c")


def runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_pins_pass_under_address_and_ub_sanitizers(tmp_path):
    asan, ubsan = runtime("libasan.so"), runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not available")
    sys.path.insert(0, ROOT)
    from oracle import build as B
    lib = tmp_path / "liboracle_san.so"
    flags = [f for f in B.CFLAGS if f != "-O2"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                  "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.run(["gcc", *flags, SRC, "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, MXFP4_ORACLE_LIB=str(lib),
               LD_PRELOAD=":".join(p for p in (asan, ubsan, os.environ.get("LD_PRELOAD", "")) if p),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
