"""include/sigattn.h from plain C: a C99 program compiled with gcc against
the header and linked with libsigattn runs the host-only calls (no GPU)."""
import os
import shutil
import subprocess

import pytest

import sigmoid_attention_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_header_compiles_as_c_and_host_calls_work(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = sa.lib_path()
    exe = str(tmp_path / "c_abi_check")
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_check.c"), lib, f"-Wl,-rpath,{os.path.dirname(lib)}",
                    "-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout
