"""CPU checks of the compiled gfx950 code (no GPU needed).

The tile kernel issues its global-to-LDS loads through inline assembly. The
compiler does not see what such a block writes, so the block may only set
M0 (declared) and issue the load; in particular it must not write SCC, which
the compiler may hold live across it (a loop condition): an undeclared SCC
write there once corrupted a loop exit test.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tile_partitioned_dense_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

# M0 may be set from any scalar register, including the VCC halves the
# allocator sometimes picks for a plain SGPR operand.
ALLOWED = re.compile(r"^(s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)|"
                     r"buffer_load_dwordx4 v\d+, s\[\d+:\d+\], (0|s\d+) offen lds)$")


@pytest.fixture(scope="module")
def tile_asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "k.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-DTG_TILE_CONFIG=1", "-S", "--cuda-device-only",
           os.path.join(CSRC, "kernels_tile.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def test_inline_asm_blocks_only_set_m0_and_load(tile_asm):
    blocks = re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", tile_asm, flags=re.S)
    assert blocks, "expected the LDS-DMA inline assembly"
    for b in blocks:
        for line in b.strip().splitlines():
            assert ALLOWED.match(line.strip()), f"unexpected instruction in inline asm: {line.strip()}"


def test_m0_written_only_by_the_dma_blocks(tile_asm):
    outside = re.sub(r";;#ASMSTART\n.*?;;#ASMEND", "", tile_asm, flags=re.S)
    writes = [l for l in outside.splitlines() if re.match(r"^\s*s_\w+\s+m0\b", l)]
    assert not writes, writes[:5]
