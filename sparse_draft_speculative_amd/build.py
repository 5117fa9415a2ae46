"""Build libstdspec.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python -m sparse_draft_speculative_amd.build   (or build() from Python)
Always recompiles every source; objects go to _build/ next to this file.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libstdspec.so")
SOURCES = ["api.hip", "attention.hip", "select.hip", "accept.hip", "probe.hip", "check.hip",
           "prefill.hip", "window.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # no packed fp32 instructions (v_pk_*_f32) in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libstdspec")
    return exe


def build(verbose=False):
    """Compile every source for gfx950 and link libstdspec.so."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        # the host pass does not know the packed-fp32 feature; that note is harmless
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB)
    return LIB


TEST_PROGRAM_SRC = os.path.join(ROOT, "tests", "cycle_from_c.hip")
TEST_PROGRAM = os.path.join(ROOT, "tests", "_build", "cycle_from_c")


def build_test_program(verbose=False):
    """The GPU test program that drives a cycle through the C ABI alone
    (tests/cycle_from_c.hip), linked against the in-tree libstdspec.so."""
    os.makedirs(os.path.dirname(TEST_PROGRAM), exist_ok=True)
    cmd = [hipcc(), *FLAGS, TEST_PROGRAM_SRC, "-L", HERE, "-lstdspec",
           "-Wl,-rpath,$ORIGIN/../../sparse_draft_speculative_amd", "-o", TEST_PROGRAM]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if res.returncode != 0:
        out = res.stdout.decode(errors="replace")
        print("\n".join(ln for ln in out.splitlines() if "packed-fp32-ops" not in ln),
              file=sys.stderr)
        raise RuntimeError("hipcc failed for tests/cycle_from_c.hip")
    return TEST_PROGRAM


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
