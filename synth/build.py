"""Builds synth/libmoe_synth.so (the GPU fill of synthetic expert records)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe_synth.so")


def build() -> str:
    cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--offload-arch=gfx950", "-O3",
           "-std=c++17", "-fPIC", "-shared", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", os.path.join(HERE, "fill.hip"), "-o", LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
