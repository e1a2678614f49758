"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* the quotient checker (plain C) and the launchers' host logic
  (``tests/csrc/host_logic_check.hip`` built by the host compiler alone);
* the C ABI's argument validation: every library source compiled with the
  sanitizers on its host side only (the device code is built as usual), the
  library linked against the clang runtime, and ``tests/test_abi.py`` run in a
  subprocess that preloads it. Every error halts the run.

No test here touches a GPU.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

import pytest

from fp8_quant_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_quant_amd", "csrc")
SOURCES = [s[: -len(".hip")] for s in build.SOURCES]  # every unit of the library
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _clean(out: subprocess.CompletedProcess) -> str:
    text = out.stdout + out.stderr
    assert "runtime error" not in text and "AddressSanitizer" not in text, text[-2000:]
    return text


def test_quotient_check_under_sanitizers(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "quotient_check"
    subprocess.run([cc, "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(ROOT, "tests", "csrc", "quotient_check.c"), "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe), "7", "0", "0", "0", str(1 << 23), "4099"], capture_output=True, text=True,
                         timeout=300, env={**os.environ, **SAN_ENV})
    _clean(out)
    assert out.returncode == 0
    total, bad = map(int, out.stdout.split())
    assert total > 0 and bad == 0


def test_host_logic_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("g++ or the HIP headers not available")
    exe = tmp_path / "host_logic_check"
    subprocess.run([cxx, "-x", "c++", "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", os.path.join(ROOT, "tests", "csrc", "host_logic_check.hip"),
                    "-o", str(exe)], check=True)
    env = {**os.environ, **SAN_ENV}
    out = subprocess.run([str(exe), "div"], capture_output=True, text=True, timeout=300, env=env)
    _clean(out)
    assert out.returncode == 0 and ", 0 wrong" in out.stdout
    out = subprocess.run([str(exe), "clamp", "448", "240", "232", "57.5", "0.5"], capture_output=True, text=True,
                         timeout=60, env=env)
    _clean(out)
    assert out.returncode == 0 and out.stdout.split()[1::2] == ["0", "0", "1", "0", "0"]


@pytest.mark.slow
def test_abi_validation_under_sanitizers(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc"
    clangxx = "/opt/rocm/lib/llvm/bin/clang++"
    rt = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not (os.path.exists(hipcc) and os.path.exists(clangxx) and rt):
        pytest.skip("hipcc, clang++ or the clang sanitizer runtime not available")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all"]
    procs = []
    for name in SOURCES:
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, name + ".hip"),
               "-o", str(tmp_path / (name + ".o"))]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out[-2000:]
    lib = tmp_path / "librnq_sanitized.so"
    subprocess.run([clangxx, "--hip-link", "--offload-arch=gfx950", "-shared", *host_san[:4], "-Xarch_host",
                    "-shared-libsan", *[str(tmp_path / (n + ".o")) for n in SOURCES], "-L/opt/rocm/lib",
                    "-lamdhip64", "-o", str(lib)], check=True)
    syms = subprocess.run(["nm", "-D", str(lib)], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms  # the host code is instrumented
    env = {**os.environ, **SAN_ENV, "LD_PRELOAD": rt[0], "RNQ_LIBRARY": str(lib)}
    out = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                          "-p", "no:cacheprovider"], capture_output=True, text=True, timeout=600, env=env, cwd=ROOT)
    text = _clean(out)
    assert out.returncode == 0, text[-3000:]
    assert " passed" in text and "failed" not in text
