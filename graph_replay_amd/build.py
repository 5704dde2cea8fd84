"""Build libstep.so (the C-ABI step and MoE library) in-tree for gfx950 with hipcc."""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "csrc", "step.hip"), os.path.join(HERE, "csrc", "moe.hip")]
OUT = os.path.join(HERE, "libstep.so")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         # keep the compiler from forming packed fp32 instructions
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    """Compile each source to an object (in parallel), then link the shared library."""
    with tempfile.TemporaryDirectory(prefix="libstep_") as tmp:
        objs, procs = [], []
        for src in SRCS:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            objs.append(obj)
            procs.append(subprocess.Popen(["hipcc", *FLAGS, "-c", "-o", obj, src], stdout=subprocess.PIPE,
                                          stderr=subprocess.PIPE, text=True))
        logs, failed = [], False
        for p in procs:
            out, err = p.communicate()
            logs.append(out + err)
            failed |= p.returncode != 0
        if not failed:
            res = subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", OUT + ".tmp", *objs],
                                 capture_output=True, text=True)
            logs.append(res.stdout + res.stderr)
            failed = res.returncode != 0
    text = "\n".join(logs)
    if failed:
        sys.stderr.write(text)
        raise RuntimeError("hipcc failed building libstep.so")
    if verbose:
        sys.stderr.write("\n".join(l for l in text.splitlines() if "packed-fp32" not in l) + "\n")
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
