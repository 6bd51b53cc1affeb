"""The library from plain C99: tests/c_abi/abi_smoke.c includes only moe.h
and the HIP runtime's C API.  On the CPU it must compile and link against
libmoe.so without warnings; on an MI355X it runs route, permute, grouped
SwiGLU forward and combine and checks the results' invariants."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "fine_grained_moe_amd")
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_smoke.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(out):
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    if not os.path.exists(os.path.join(LIBDIR, "libmoe.so")):
        pytest.skip("libmoe.so not built")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", SRC, f"-L{LIBDIR}", "-lmoe",
           f"-L{ROCM}/lib", "-lamdhip64", "-lm", f"-Wl,-rpath,{LIBDIR}", f"-Wl,-rpath,{ROCM}/lib",
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr


def test_c_program_builds(tmp_path):
    _build(str(tmp_path / "abi_smoke"))


@pytest.mark.gpu
def test_c_program_runs(tmp_path):
    exe = str(tmp_path / "abi_smoke")
    _build(exe)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert "c-abi ok" in r.stdout
