"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer: the
pin suites run again, in a child process, against a build of oracle/pkv_oracle.c
instrumented with both (gcc, host code only), and must pass with no report.  The
oracle is the parity tests' ground truth, so a read past a buffer or an overflow
in it would go unseen by the pins alone."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_slotted.py",
          "tests/test_oracle_cow.py", "tests/test_oracle_slot_cow.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_pins_clean_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = str(tmp_path / "libpkv_oracle_sanitized.so")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                    "-fno-fast-math", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-o", lib, os.path.join(ROOT, "oracle", "pkv_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, PKV_ORACLE_LIB=lib, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *SUITES], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
