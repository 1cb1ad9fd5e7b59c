"""The C ABI from a C11 caller: tests/c/abi_host.c is compiled against
include/ddpb.h with gcc -std=c11 -pedantic -Werror, linked to the host-only
library (same plan and state machine, no device work) and run."""
import os
import shutil
import subprocess

import pytest

import ddp_bucketed_gradient_amd as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_against_the_header(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(D.HOSTONLY_LIB):
        from ddp_bucketed_gradient_amd import build
        build.build_hostonly()
    exe = tmp_path / "abi_host"
    libdir = os.path.dirname(D.HOSTONLY_LIB)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_host.c"),
                    D.HOSTONLY_LIB, f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "c abi ok"
