"""AddressSanitizer build of the C ABI's host code (api.cpp), driven on the CPU.

api.cpp is compiled with the sanitizer on its host side only (its device code, a fill
kernel, is built as usual) and linked with the library's other objects into
tests/asan/abi_host_driver.cpp, which calls every entry point of include/moe.h on
arguments its validation rejects and checks each status.  No call reaches a HIP launch,
so no GPU is needed; any out-of-bounds or use-after-free access in the validation and
workspace arithmetic ends the run with the sanitizer's report."""
import os
import subprocess

import pytest

from mixture_experts_layer_33_amd import build as libbuild

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(libbuild.BUILD, "asan")
OTHER_OBJS = [os.path.splitext(s)[0] + ".o" for s in libbuild.SOURCES if s != "api.cpp"]

# -fsanitize applies to the host pass only (-Xarch_host before each sanitizer option)
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_api_host_code_under_address_sanitizer():
    objs = [os.path.join(libbuild.BUILD, o) for o in OTHER_OBJS]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        libbuild.build()
    os.makedirs(OUT, exist_ok=True)
    api_o = os.path.join(OUT, "api_asan.o")
    drv_o = os.path.join(OUT, "driver_asan.o")
    exe = os.path.join(OUT, "abi_host_driver")
    base = [libbuild.HIPCC, "-O1", "-g", "-std=c++17", f"--offload-arch={libbuild.ARCH}",
            "-I", libbuild.INCLUDE, "-I", libbuild.CSRC, "-Wno-unused-command-line-argument",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    run(base + HOST_ASAN + ["-x", "hip", "-c", os.path.join(libbuild.CSRC, "api.cpp"), "-o", api_o])
    run(base + HOST_ASAN + ["-c", os.path.join(HERE, "asan", "abi_host_driver.cpp"), "-o", drv_o])
    run([libbuild.HIPCC, f"--offload-arch={libbuild.ARCH}", "-Xarch_host", "-fsanitize=address",
         "-o", exe, drv_o, api_o] + objs)
    env = dict(os.environ)
    # the HIP runtime keeps its code-object registrations until exit: not leaks of api.cpp
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert "AddressSanitizer" not in r.stderr
    assert r.returncode == 0 and "ok: 0 failure(s)" in r.stdout
