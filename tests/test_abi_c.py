"""The header is usable from C: `include/hybrid_swa_kv.h` compiles as strict C99
and C11 (and as C++17), and a C program linked against the built library gets
the documented status codes from the host-side checks (tests/c/abi_from_c.c).
CPU only: every call it makes is rejected before any device work."""

import os
import shutil
import subprocess

import pytest

from hybrid_swa_kv_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "include")
SRC = os.path.join(ROOT, "tests", "c", "abi_from_c.c")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


@pytest.mark.parametrize("std", ["c99", "c11"])
def test_header_compiles_as_c(std, tmp_path):
    r = subprocess.run(["gcc", f"-std={std}", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-x", "c", os.path.join(INC, "hybrid_swa_kv.h")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_header_compiles_as_cxx():
    r = subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-x", "c++", os.path.join(INC, "hybrid_swa_kv.h")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_gets_documented_status_codes(tmp_path):
    if not os.path.exists(_lib.LIB_PATH):
        from hybrid_swa_kv_amd import build

        build.build()
    libdir = os.path.dirname(os.path.abspath(_lib.LIB_PATH))
    exe = str(tmp_path / "abi_from_c")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", INC, SRC, "-o", exe,
                        os.path.abspath(_lib.LIB_PATH), f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
