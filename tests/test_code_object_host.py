"""The gfx950 code objects of the built library, read from their metadata notes:
every kernel keeps its state in registers and LDS (no scratch memory, whose
per-lane traffic would compete with the cache streams for HBM), and the split
kernel's instantiations cover what the launchers dispatch."""

import os
import re
import shutil
import subprocess

import pytest

from decode_attention_int4_block_amd import _lib

LLVM = "/opt/rocm/llvm/bin"


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    objdump, readelf = os.path.join(LLVM, "llvm-objdump"), os.path.join(LLVM, "llvm-readelf")
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libkvq.so not built")
    if not (os.path.exists(objdump) and os.path.exists(readelf)):
        pytest.skip("llvm tools not found")
    d = tmp_path_factory.mktemp("co")
    shutil.copy(_lib.LIB_PATH, d / "libkvq.so")
    subprocess.run([objdump, "--offloading", "libkvq.so"], cwd=d, check=True, capture_output=True)
    found = {}
    for f in sorted(os.listdir(d)):
        if "amdgcn-amd-amdhsa--gfx950" not in f:
            continue
        notes = subprocess.run([readelf, "--notes", str(d / f)], check=True, capture_output=True, text=True).stdout
        name = None
        for line in notes.splitlines():
            m = re.match(r"\s*\.name:\s+(\S+)", line)
            if m:
                name = m.group(1)
            m = re.match(r"\s*\.private_segment_fixed_size:\s+(\d+)", line)
            if m and name:
                found[name] = int(m.group(1))
                name = None
    assert found, "no gfx950 kernels found in the library"
    return found


def test_no_kernel_uses_scratch(kernels):
    spilled = {k: v for k, v in kernels.items() if v != 0}
    assert not spilled, f"kernels with scratch: {spilled}"


def test_split_kernel_instantiations(kernels):
    split = [k for k in kernels if "decode_split_kernel" in k]
    # 3 group classes x (attention, fused) x 3 widths, the read skeletons,
    # and the grouped-key kernels (2 group classes x 3 widths)
    assert len(split) >= 18 + 6
    assert any("prefill_kernel" in k for k in kernels)
    assert any("decode_combine_kernel" in k for k in kernels)
    assert sum("quant_append_kernel" in k for k in kernels) == 6
