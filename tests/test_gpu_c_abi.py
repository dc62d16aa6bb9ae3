"""The C ABI used from plain C: tests/c_abi_check.c (built next to the library)
calls paged_attention_append_decode, paged_attention_decode and
paged_attention_append_decode_slotted through include/paged_kv.h with device
memory from the HIP runtime, no Python in between, and checks closed-form
results (one-token contexts, by block table or by slotted segment, return the
appended value row bit for bit; scale 0 returns the mean of the value rows) and
status codes."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi_check")


@pytest.mark.gpu
def test_c_program_drives_the_abi():
    assert os.path.exists(BIN), "tests/c_abi_check is not built: python -m paged_kv_cache_09_amd.build"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 4 and all(": ok" in ln for ln in lines), r.stdout
