"""Builds ``libmoe_tail.so`` (the tail) and ``libmoe_tail_probes.so`` (the
measurement probes) in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "moe_tail.hip")
OUT = os.path.join(HERE, "libmoe_tail.so")
PROBES_SRC = os.path.join(HERE, "csrc", "probes.hip")
PROBES_OUT = os.path.join(HERE, "libmoe_tail_probes.so")

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


def _hipcc(src: str, out: str) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    subprocess.run([hipcc, *HIPCC_FLAGS, src, "-o", tmp], check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    _hipcc(PROBES_SRC, PROBES_OUT)
    return _hipcc(SRC, OUT)


if __name__ == "__main__":
    print(build())
