"""Builds libdustin.so (the gfx950 HIP library behind include/dustin.h) in-tree."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libdustin.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 VALU ops stay off (only plain fp32 arithmetic is emitted)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (avoids accumulator-register copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libdustin.so (always recompiles)."""
    objs = []
    procs = []
    for src in sources():
        obj = os.path.join(CSRC, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = "\n".join(l for l in out.decode(errors="replace").splitlines()
                         if "packed-fp32-ops" not in l)
        if text.strip():
            print(text, file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    subprocess.check_call([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    for o in objs:
        os.remove(o)
    return LIB_PATH


EXAMPLE_SRC = os.path.join(ROOT, "tests", "c_abi_example.c")
EXAMPLE_BIN = os.path.join(ROOT, "tests", "c_abi_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_example(verbose: bool = False) -> str:
    """The C program under tests/ that calls libdustin.so through dustin.h alone (plain C,
    the HIP runtime for device memory); found next to the library through its rpath."""
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(ROCM, "include"), EXAMPLE_SRC, "-o", EXAMPLE_BIN,
           "-L", PKG, "-ldustin", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../sparse_kv_attention_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    return EXAMPLE_BIN


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_example(verbose=True))
