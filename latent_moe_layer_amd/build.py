"""Builds ``libmoe_tail.so`` in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "moe_tail.hip")
OUT = os.path.join(HERE, "libmoe_tail.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # no packed-FP32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: with the accumulation-register form
    # the compiler copies the accumulators between the two register files on
    # every K step of the small-M dense loop
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*"))) + \
        [os.path.join(os.path.dirname(HERE), "include", "moe_tail.h")]


def build() -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = OUT + ".tmp"
    subprocess.run([hipcc, *HIPCC_FLAGS, SRC, "-o", tmp], check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
