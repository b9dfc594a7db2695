"""Compile libmoe.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

Run as a script (python mixture_experts_layer_f32_amd/build.py) or through
__graft_entry__.build(); importing the package itself requires the library."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = [os.path.join(HERE, "csrc", "moe_api.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # packed-f32 VALU forms stay off (the compiler may otherwise emit them from float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I" + os.path.join(ROOT, "include"),
                                     "-I" + os.path.join(HERE, "csrc")] + SOURCES + ["-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
