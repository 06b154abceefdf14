"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle.c is rebuilt with -fsanitize=address,undefined (host code only; gcc,
no GPU code involved) and the pin suite runs against that build, the
sanitizer runtime preloaded into the test process.  Any out-of-bounds read of
a padded operand, use of freed scratch memory, signed overflow in an index or
other undefined behaviour aborts the run, so the oracle's results are not
merely right on these inputs but come from well-defined accesses."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")


def _runtime(name):
    r = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_pins_pass_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-fPIC", "-shared",
                    "-ffp-contract=off", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-o", str(lib), SRC], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="2", LD_PRELOAD=asan,
               # the interpreter's own allocations are not the oracle's: no leak report
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, out


@pytest.mark.slow
def test_sanitizer_build_reports_a_planted_overread(tmp_path):
    """Control: the same build and runtime do report an access one element
    past a buffer (planted in a copy of the oracle's fp16 decode loop), so
    the passing run above is not a sanitizer that never fires."""
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    text = open(SRC).read()
    old = "for (long t = 0; t < count; ++t)\n        out[t] = oracle_half_to_double(h[t]);"
    assert old in text
    src = tmp_path / "overread.c"
    src.write_text(text.replace(old, "for (long t = 0; t <= count; ++t)\n        out[t] = "
                                     "oracle_half_to_double(h[t]);"))
    lib = tmp_path / "liboverread.so"
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", str(lib),
                    str(src)], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0")
    code = ("import numpy as np, oracle; "
            "oracle.half_to_double(np.arange(1000, dtype=np.uint16))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stderr[-2000:]
