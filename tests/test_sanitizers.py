"""The CPU oracle and the host side of the tail's C ABI built with the
address and undefined-behaviour sanitizers and run on the CPU
(tests/sanitize/*.cpp drive them).  The ABI build compiles the library
sources with the sanitizers on the host pass only; no device code runs."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(exe, extra_env):
    env = dict(os.environ)
    env.update(extra_env)
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    os.path.join(HERE, "oracle_driver.cpp"), "-o", exe], check=True, timeout=600)
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=1", "OMP_NUM_THREADS": "2"})
    assert "oracle driver: ok" in out


def test_abi_host_side_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("no hipcc")
    exe = str(tmp_path / "abi_driver")
    src = os.path.join(ROOT, "latent_moe_layer_amd", "csrc")
    # the sanitizers on the host pass only: each -fsanitize= right after -Xarch_host
    # (device code as the library builds it; the host pass at -O1 with debug info)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Xarch_host", "-O1", "-Xarch_host", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           os.path.join(HERE, "abi_driver.cpp"), os.path.join(src, "moe_tail.hip"), os.path.join(src, "probes.hip"),
           "-o", exe]
    subprocess.run(cmd, check=True, timeout=900, capture_output=True)
    # (the HIP runtime keeps allocations until exit: leak reports would be its own)
    out = _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
    assert "abi driver: ok" in out
