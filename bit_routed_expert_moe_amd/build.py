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
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # MFMA results straight into VGPRs (no AGPR round trip before the
         # fp32 group epilogue of the grouped kernels)
         "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function"]
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if NOISE not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(extra: list[str] | None = None, out: str = LIB) -> str:
    """Compiles every source to an object in parallel, then links the library."""
    import concurrent.futures as cf
    import tempfile
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmp:
        objs = [os.path.join(tmp, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, *(extra or []), "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with cf.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for f in [ex.submit(_run, c) for c in cmds]:
                f.result()
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *(extra or []), *objs, "-o", out])
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
