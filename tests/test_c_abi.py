"""The boundary from C: tests/c_abi_client.c includes include/csa.h, is
compiled by the system C compiler, links the built libcsa.so and checks the
host side of the entry points (no GPU: every call is refused before a
launch)."""
import os
import shutil
import subprocess

import pytest

from compressed_sparse_long_csa_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_client_compiles_links_and_passes(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libcsa.so is not built")
    libdir = os.path.dirname(binding.LIB_PATH)
    exe = str(tmp_path / "c_abi_client")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "c_abi_client.c"), "-L", libdir, "-lcsa",
                        f"-Wl,-rpath,{libdir}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi ok" in r.stdout
