"""Builds libpirscan.so in-tree (hipcc for gfx950, via the csrc Makefile)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(force: bool = True, jobs: int = 4) -> str:
    cmd = ["make", "-C", os.path.join(HERE, "csrc"), f"-j{jobs}"] + (["-B"] if force else [])
    subprocess.run(cmd, check=True)
    return os.path.join(HERE, "libpirscan.so")


if __name__ == "__main__":
    print(build())
