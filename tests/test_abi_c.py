"""The C ABI used from C: tests/abi_from_c.c includes only include/stdspec.h
(compiled as C11 by gcc), links libstdspec.so and runs host-side checks of
every call of the hot path (each stopped before any launch, so no GPU is
needed)."""

import os
import shutil
import subprocess

import pytest

from sparse_draft_speculative_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH) or not shutil.which("gcc"),
                                reason="libstdspec.so not built or no gcc")


def test_header_compiles_as_c_and_calls_reject_on_the_host(tmp_path):
    exe = tmp_path / "abi_from_c"
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "abi_from_c.c"),
                    "-L", libdir, "-lstdspec", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                   check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failure(s)" in res.stdout
