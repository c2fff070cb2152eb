"""The library's host code (csrc/mla_api.cpp: validation, split planning,
workspace sizing, error reporting) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

tests/sanitize/abi_host_driver.cpp is linked with the API source compiled
with host-side sanitizers (device code, the allocation-free entry point's
scratch array only, is built without them) and with stub kernel launchers
that abort, so no check can reach a kernel.  The driver runs every
rejection clause of every entry point, zero-token calls, sweeps of the
host-only planners over extreme values, and thread-local error messages
from eight threads.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "head_latent_attention_sparse_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_host_driver.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"

# Sanitizers for the host pass only; the device pass of these files holds
# no code that runs here.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
LINK_SANITIZE = ["-fsanitize=address", "-fsanitize=undefined"]


def _compile(src, obj):
    cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-x", "hip", "-c", src, "-o", obj,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *HOST_SANITIZE]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr


def test_host_abi_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("the ROCm compilers are not installed")
    api_obj, drv_obj, exe = tmp_path / "mla_api.o", tmp_path / "driver.o", tmp_path / "abi_host_driver"
    _compile(os.path.join(CSRC, "mla_api.cpp"), str(api_obj))
    _compile(DRIVER, str(drv_obj))
    link = [CLANGXX, *LINK_SANITIZE, str(drv_obj), str(api_obj), "-o", str(exe), "-L/opt/rocm/lib", "-lamdhip64",
            "-Wl,-rpath,/opt/rocm/lib", "-pthread"]
    r = subprocess.run(link, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # host paths only, also where a GPU is present
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
