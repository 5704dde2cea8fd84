"""Build libstep.so (the C-ABI step library) in-tree for gfx950 with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "step.hip")
OUT = os.path.join(HERE, "libstep.so")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         # keep the compiler from forming packed fp32 instructions
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    cmd = ["hipcc", *FLAGS, "-o", OUT + ".tmp", SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libstep.so")
    if verbose:
        sys.stderr.write("\n".join(l for l in res.stderr.splitlines() if "packed-fp32" not in l) + "\n")
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
