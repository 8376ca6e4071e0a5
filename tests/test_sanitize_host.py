"""Host sanitizer runs (CPU only): the oracle, and the C-ABI library's host
code, built with AddressSanitizer and UndefinedBehaviorSanitizer (no
recovery) and driven by the programs under tests/sanitize/.  The library's
device code is linked from the normal build, uninstrumented: GPU sanitizers
are not part of this (the drivers make no GPU call)."""
import os
import pathlib
import shutil
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
SAN = ROOT / "tests" / "sanitize"
OBJ = ROOT / "_build" / "obj"
DEVICE_OBJECTS = ["quant_kernels.hip.o", "gemm_kernels.hip.o", "gemm_tiled.hip.o",
                  "gemm_skinny.hip.o", "moe_epilogue.hip.o", "noalloc.hip.o"]
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, (cmd[0], r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
         f"-I{ROOT / 'oracle'}", str(ROOT / "oracle" / "mxfp4_oracle.c"),
         str(SAN / "oracle_driver.c"), "-o", str(exe), "-lm"])
    r = run([str(exe)], env=ENV)
    assert "oracle sanitizer run ok" in r.stdout


HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
# every sanitizer flag applies to the host side of the compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not pathlib.Path(HIPCC).exists(), reason="no hipcc")
def test_library_host_code_under_address_and_undefined_sanitizers(tmp_path):
    if not all((OBJ / o).exists() for o in DEVICE_OBJECTS):
        run([sys.executable, str(ROOT / "w4a4_mxfp4_gemm_amd" / "build.py")])
    inc = [f"-I{ROOT / 'include'}", f"-I{ROOT / 'w4a4_mxfp4_gemm_amd' / 'csrc'}"]
    objs = []
    for src in (ROOT / "w4a4_mxfp4_gemm_amd" / "csrc" / "mxfp4_abi.cpp",
                ROOT / "w4a4_mxfp4_gemm_amd" / "csrc" / "layerwise.cpp",
                SAN / "abi_driver.cpp"):
        o = tmp_path / (src.name + ".o")
        run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SAN, *inc, "-c", str(src), "-o", str(o)])
        objs.append(str(o))
    exe = tmp_path / "abi_driver"
    run([HIPCC, "--offload-arch=gfx950", *HOST_SAN, *objs, *[str(OBJ / o) for o in DEVICE_OBJECTS],
         "-o", str(exe)])
    # the HIP runtime's own allocations outlive main: leaks are not checked
    env = dict(ENV, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0")
    r = run([str(exe)], env=env)
    assert "library host sanitizer run ok" in r.stdout
