"""The oracle's pins once more, with the oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no GPU).  Any out-of-bounds access,
use after free or undefined operation in oracle.c aborts the child run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.timeout(600)
def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from oracle import oracle as O

    lib = str(tmp_path / "liboracle_san.so")
    O.build(force=True, sanitize=True, out=lib)
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=580)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    # the instrumentation is live: a planted overflow (the 256-entry fp8 table written
    # into a 128-entry buffer) is reported and aborts
    probe = ("import ctypes, numpy as np; L = ctypes.CDLL(%r); "
             "b = np.zeros(128); L.orc_fp8_table(ctypes.c_void_p(b.ctypes.data))" % lib)
    r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
