"""CPU checks of the built library's own gfx950 code objects.

Every HIP source is compiled with packed FP32 turned off (the device pass
honours -Xclang -target-feature -Xclang -packed-fp32-ops; only the host pass
warns that it does not know the feature). These tests disassemble the code
objects inside libfp8blk.so and check that:
  - no packed FP32 add, multiply or fused multiply-add was emitted;
  - no kernel spills registers to scratch memory (a spill silently turns a
    bandwidth-bound kernel into one that also writes and re-reads scratch).
"""
import glob
import os
import re
import shutil
import subprocess
import tempfile

import pytest

import block_scaled_fp8_fp8blk_amd as fb

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
READELF = "/opt/rocm/llvm/bin/llvm-readelf"


@pytest.fixture(scope="module")
def code_objects():
    if not (os.path.exists(OBJDUMP) and os.path.exists(READELF)):
        pytest.skip("ROCm LLVM tools not available")
    if not os.path.exists(fb.LIB_PATH):
        pytest.fail(f"{fb.LIB_PATH} is not built")
    tmp = tempfile.mkdtemp()
    try:
        lib = shutil.copy(fb.LIB_PATH, os.path.join(tmp, "lib.so"))
        subprocess.run([OBJDUMP, "--offloading", lib], check=True, capture_output=True, cwd=tmp)
        objs = sorted(glob.glob(os.path.join(tmp, "lib.so.*gfx950")))
        assert objs, "no gfx950 code object in the library"
        yield [(o, open(o, "rb").read()) for o in objs]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_no_packed_fp32_instructions(code_objects):
    bad = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
    for path, _ in code_objects:
        asm = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", path], check=True, capture_output=True,
                             text=True).stdout
        assert "v_mfma" in asm or "k_" in asm  # the disassembly is real
        hits = bad.findall(asm)
        assert not hits, f"{os.path.basename(path)}: {len(hits)} packed FP32 instructions"


def test_no_kernel_spills_to_scratch(code_objects):
    kernels = 0
    for path, _ in code_objects:
        notes = subprocess.run([READELF, "--notes", path], check=True, capture_output=True, text=True).stdout
        symbols = re.findall(r"\.symbol:\s+(\S+)\.kd", notes)
        sizes = [int(v) for v in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", notes)]
        assert len(sizes) == len(symbols) > 0, os.path.basename(path)
        spilled = [k for k, sz in zip(symbols, sizes) if sz]
        assert not spilled, f"kernels with scratch: {spilled}"
        kernels += len(sizes)
    assert kernels >= 20
