"""The oracle's pins again, with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

An out-of-bounds access, a use of freed memory, a signed overflow or a bad shift in
jt_oracle.c aborts the child process instead of passing silently.  The child runs every
tests/test_oracle_*.py file with the sanitized library loaded through JT_ORACLE_LIB and
the sanitizer runtimes preloaded (the Python interpreter itself is not instrumented;
leak checking is off because the interpreter keeps memory until exit).
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _runtime(name):
    cc = shutil.which("gcc")
    if cc is None:
        return None
    path = subprocess.run([cc, f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = oracle.build_sanitized(str(tmp_path / "libjt_oracle_san.so"))
    env = dict(os.environ)
    env.update(JT_ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    pins = sorted(glob.glob(os.path.join(HERE, "test_oracle_*.py")))
    pins = [p for p in pins if not p.endswith("test_oracle_sanitized.py")]
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                          "-p", "no:cacheprovider", *pins], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
