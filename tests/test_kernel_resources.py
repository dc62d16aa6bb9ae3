"""Resource use of the built kernels, read from the gfx950 code objects inside
libpagedkv.so (host only, no GPU).

Every kernel must run without scratch memory.  Beyond the cost of spills, the
shared-prefix and slotted-tile kernels count their global-to-LDS loads with
explicit vector-memory waits: a scratch access inside their step loop would
enter the same in-order counter and let a wave read a staging buffer before its
data has landed.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "..", "paged_kv_cache_09_amd", "libpagedkv.so")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _tool(name):
    path = os.path.join(LLVM, name)
    return path if os.path.exists(path) else shutil.which(name)


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    tools = {n: _tool(n) for n in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")}
    if not os.path.exists(LIB) or not all(tools.values()):
        pytest.skip("built library or ROCm LLVM tools not present")
    tmp = tmp_path_factory.mktemp("codeobj")
    fat = tmp / "fatbin.bin"
    subprocess.run([tools["llvm-objcopy"], "-O", "binary", "--only-section=.hip_fatbin", LIB,
                    str(fat)], check=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    assert starts, "no offload bundle in .hip_fatbin"
    out = {}
    for i, s in enumerate(starts):
        part = tmp / f"bundle{i}.bin"
        part.write_bytes(data[s:starts[i + 1] if i + 1 < len(starts) else len(data)])
        co = tmp / f"co{i}.o"
        subprocess.run([tools["clang-offload-bundler"], "--unbundle", "--type=o",
                        f"--input={part}", f"--targets={TARGET}", f"--output={co}"], check=True)
        notes = subprocess.run([tools["llvm-readelf"], "--notes", str(co)], check=True,
                               capture_output=True, text=True).stdout
        name = None
        for line in notes.splitlines():
            m = re.match(r"\s+\.name:\s+(\S+)", line)
            if m:
                name = m.group(1)
                out[name] = {}
                continue
            m = re.match(r"\s+\.(private_segment_fixed_size|vgpr_count|group_segment_fixed_size):"
                         r"\s+(\d+)", line)
            if m and name is not None:
                out[name][m.group(1)] = int(m.group(2))
    return out


def test_code_objects_hold_every_kernel_family(kernels):
    names = " ".join(kernels)
    for family in ("decode_g1_kernel", "decode_mfma_kernel", "prefix_fused_mfma_kernel",
                   "prefix_mfma_kernel", "slotted_tiled_mfma_kernel", "slotted_mfma_kernel",
                   "reduce_kernel"):
        assert family in names, family


def test_no_kernel_uses_scratch(kernels):
    spilled = {k: v["private_segment_fixed_size"] for k, v in kernels.items()
               if v.get("private_segment_fixed_size", 0) != 0}
    assert not spilled, f"kernels with scratch memory: {spilled}"


def test_staged_kernels_fit_their_occupancy(kernels):
    # two waves per SIMD: at most 256 VGPRs, and one work-group's LDS per CU
    for k, v in kernels.items():
        if "prefix_fused_mfma_kernel" in k or "slotted_tiled_mfma_kernel" in k:
            assert v["vgpr_count"] <= 256, (k, v)
            assert v["group_segment_fixed_size"] <= 160 * 1024, (k, v)
