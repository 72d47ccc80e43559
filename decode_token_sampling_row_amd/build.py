"""Build the HIP sampler library (gfx950) in-tree with hipcc.

    python -m decode_token_sampling_row_amd.build

produces ``decode_token_sampling_row_amd/libsampler.so`` from the sources in
``csrc/`` and the public header in ``include/``.  Every call recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsampler.so")
ARCH = os.environ.get("SAMPLER_OFFLOAD_ARCH", "gfx950")

# Device code: IEEE-correct fp32 division, denormals kept, no contraction of
# separately written multiplies and adds, and no packed-fp32 instructions.
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP sampler library cannot be built")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    inc = ["-I", INCLUDE, "-I", CSRC]
    with tempfile.TemporaryDirectory() as tmp:
        k_obj = os.path.join(tmp, "sampler_kernels.o")
        a_obj = os.path.join(tmp, "sampler_api.o")
        cmds = [
            [cc, *DEVICE_FLAGS, *inc, "-x", "hip", "-c",
             os.path.join(CSRC, "sampler_kernels.hip"), "-o", k_obj],
            [cc, *DEVICE_FLAGS, *inc, "-c", os.path.join(CSRC, "sampler_api.cpp"), "-o", a_obj],
        ]
        tmp_lib = LIB + ".tmp"
        cmds.append([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", k_obj, a_obj, "-o", tmp_lib])
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
