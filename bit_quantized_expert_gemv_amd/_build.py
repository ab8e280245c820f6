"""Build libbqmoe.so (the C-ABI library with its gfx950 kernels) in place with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbqmoe.so")

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
SOURCES = ["moe_host.cpp", "moe_kernels.hip", "moe_prefill.hip"]


def build(verbose: bool = False) -> str:
    cmd = ["hipcc", *HIP_FLAGS, *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB]
    if verbose:
        print(" ".join(cmd))
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"libbqmoe build failed:\n{out}")
    if verbose and out.strip():
        print(out)
    return LIB
