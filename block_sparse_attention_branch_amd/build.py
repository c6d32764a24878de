"""Compile libmsa.so for gfx950 in-tree (make over csrc/, hipcc cross-compiles
without a GPU)."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build(jobs: int = 8, force: bool = True) -> str:
    csrc = os.path.join(HERE, "csrc")
    if force:
        subprocess.run(["make", "-C", csrc, "clean"], check=True, stdout=subprocess.DEVNULL)
    subprocess.run(["make", "-C", csrc, f"-j{jobs}", "SHELL=/bin/bash"], check=True)
    lib = os.path.join(HERE, "libmsa.so")
    if not os.path.exists(lib):
        raise RuntimeError("libmsa.so was not produced")
    return lib


if __name__ == "__main__":
    print(build())
