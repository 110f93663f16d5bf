"""Builds libmoe_layer.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_layer.so")
SOURCES = ["moe_kernels.hip", "moe_prefill.hip", "moe_stream.hip", "moe_layer.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA results straight into VGPRs (no AGPR round trip before the
         # fp32 group epilogue of the grouped kernels)
         "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function"]


def build(extra: list[str] | None = None, out: str = LIB) -> str:
    cmd = [HIPCC, *FLAGS, *(extra or []), *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
