"""The LDS-DMA loads are issued from inline asm that sets M0 itself and does
not save it.  That is only sound while the compiler keeps nothing of its own
in M0 in these kernels: check the gfx950 assembly (built here, no GPU needed)
for any M0 access other than the load sequence."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fine_grained_moe_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["grouped_gemm.hip", "router.hip"])
def test_m0_only_in_dma_sequence(tmp_path, src):
    out = tmp_path / (src + ".s")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
                    "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)],
                   check=True, capture_output=True)
    lines = [l.split(";")[0].strip() for l in out.read_text().splitlines()]
    code = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    n_dma = 0
    for i, l in enumerate(code):
        if not re.search(r"\bm0\b", l):
            continue
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", l), f"unexpected M0 use: {l}"
        assert code[i + 1] == "s_nop 0", code[i + 1]
        assert code[i + 2].startswith("buffer_load_dwordx4") and code[i + 2].endswith(" lds"), code[i + 2]
        n_dma += 1
    assert n_dma > 0
