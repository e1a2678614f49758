"""Build of tests/csrc/c_client.c, a plain C99 client of the C ABI: it includes
only include/rnq.h and the HIP runtime's C API and links librnq.so (built
first). The binary lands in tests/bin/c_client; __graft_entry__.build() builds
it with the library."""

from __future__ import annotations

import os
import shutil
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "csrc", "c_client.c")
EXE = os.path.join(ROOT, "tests", "bin", "c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = ["-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__"]


def command(out: str = EXE) -> list:
    return [shutil.which("gcc") or "gcc", *FLAGS, "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(ROCM, "include"), SRC, "-o", out,
            "-L", os.path.join(ROOT, "fp8_quant_amd"), "-lrnq", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            "-Wl,-rpath," + os.path.join(ROOT, "fp8_quant_amd"), "-Wl,-rpath,$ORIGIN/../../fp8_quant_amd",
            "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def build(out: str = EXE) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    pr = subprocess.run(command(out), stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if pr.returncode != 0:
        raise RuntimeError(f"c_client build failed:\n{pr.stdout}")
    return out
