"""Build librnq.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: ``python -m fp8_quant_amd.build`` (or ``build()`` from Python). Always
recompiles. The library lands next to this file as ``librnq.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librnq.so")
SOURCES = ["rnq_api.hip", "rnq_rows.hip", "rnq_rows_quant.hip", "rnq_rows_norm.hip", "rnq_rows_pos.hip", "rnq_wide.hip", "rnq_group.hip", "rnq_narrow_bwd.hip", "rnq_row_bwd.hip", "rnq_baselines.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",  # every multiply and add rounds on its own (no implicit FMA)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 14 dwords of kernel arguments arrive in scalar registers at wave
    # launch (gfx950 preloading): kernels whose leading arguments are scalars
    # issue their first loads without a load of the kernel arguments
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the rnq HIP library cannot be built")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        if pr.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def build_test_programs(verbose: bool = False) -> list:
    """Test-only HIP programs under tests/csrc (built next to the tests in tests/bin)."""
    cc = hipcc()
    src_dir = os.path.join(ROOT, "tests", "csrc")
    out_dir = os.path.join(ROOT, "tests", "bin")
    os.makedirs(out_dir, exist_ok=True)
    built = []
    for name in ("row_scalar_check", "host_logic_check"):
        exe = os.path.join(out_dir, name)
        cmd = [cc, *[f for f in HIPCC_FLAGS if f != "-fPIC"], "-I", INCLUDE, "-I", CSRC,
               os.path.join(src_dir, name + ".hip"), "-o", exe]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        built.append(exe)
    return built


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_test_programs(verbose="-v" in sys.argv))
