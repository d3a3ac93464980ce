"""Host-only AddressSanitizer build of the weight packer (`pack.cpp`) and the C entry points'
argument validation (`api.hip`, host code instrumented; device code built as usual), linked
with the library's other objects and driven by `tests/asan_driver.c` on the CPU: packing at
exact buffer sizes for every weight type, and the validation paths of every entry point.
Needs hipcc and g++ (no GPU); the other objects come from the in-tree build."""
import os
import shutil
import subprocess

import pytest

from quantized_expert_layer_amd import build as qbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_expert_layer_amd", "csrc")
BUILD = os.path.join(ROOT, "quantized_expert_layer_amd", "_build")
INCLUDE = os.path.join(ROOT, "include")


@pytest.mark.timeout(600)
def test_packer_and_validation_under_asan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not shutil.which("g++"):
        pytest.skip("hipcc and g++ are needed")
    others = [os.path.join(BUILD, f) for f in sorted(os.listdir(BUILD))
              if f.endswith(".o") and f not in ("api.hip.o", "pack.cpp.o")] \
        if os.path.isdir(BUILD) else []
    if len(others) < 8:
        pytest.skip("the library's objects are not built (run quantized_expert_layer_amd.build)")
    t = str(tmp_path)
    run = lambda cmd: subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=550)
    # host code of api.hip with ASan; its device code is built as in the library
    run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "api.hip"), "-o", f"{t}/api.o"])
    run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-fsanitize=address", "-fno-omit-frame-pointer",
         "-I", INCLUDE, "-c", os.path.join(CSRC, "pack.cpp"), "-o", f"{t}/pack.o"])
    run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address", "-fno-omit-frame-pointer",
         "-I", INCLUDE, "-c", os.path.join(ROOT, "tests", "asan_driver.c"), "-o", f"{t}/driver.o"])
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "lib")
    run(["g++", "-fsanitize=address", "-o", f"{t}/asan_driver", f"{t}/driver.o", f"{t}/api.o",
         f"{t}/pack.o", *others, f"-L{rocm_lib}", "-lamdhip64", "-lpthread",
         f"-Wl,-rpath,{rocm_lib}"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               HIP_VISIBLE_DEVICES=os.environ.get("HIP_VISIBLE_DEVICES", ""))
    r = subprocess.run([f"{t}/asan_driver"], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and "AddressSanitizer" not in r.stderr, r.stderr[-3000:]
    assert "all checks passed" in r.stdout
