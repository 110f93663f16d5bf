"""Builds oracle/libmoe_oracle.so from moe_oracle.c with gcc (test infrastructure).

Flags keep the arithmetic as written: no fast-math and no fused multiply-add
contraction, so every sum is evaluated in source order in IEEE double.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra: list[str] | None = None) -> str:
    cmd = ["gcc", *CFLAGS, *(extra or []), src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(extra=sys.argv[1:]))
