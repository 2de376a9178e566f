"""Builds the test-support native code (not part of libfp.so): the FP8 MFMA
probe that tests/test_gpu_fp8_mfma.py runs.  Every call recompiles."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
PROBE_SRC = os.path.join(HERE, "fp8_mfma_probe.hip")
PROBE_LIB = os.path.join(HERE, "libfp8_mfma_probe.so")


def build() -> str:
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build())
