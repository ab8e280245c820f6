"""Build libbqmoe.so (the C-ABI library with its gfx950 kernels) in place with hipcc: each source is
compiled to an object in parallel, then the objects are linked."""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbqmoe.so")
OBJ = os.path.join(HERE, "_build")

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # leading scalar kernel arguments (up to eight) preloaded into SGPRs at wave launch, so
             # the decode kernels' first loads wait for no kernel-argument fetch
             "-mllvm", "-amdgpu-kernarg-preload-count=8",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC]
SOURCES = ["moe_host.cpp", "moe_kernels.hip", "moe_prefill.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out, cmd


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(OBJ, exist_ok=True)
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    cmds = [["hipcc", *HIP_FLAGS, *extra_flags, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(len(cmds)) as ex:
        results = list(ex.map(_run, cmds))
    for rc, out, cmd in results:
        if verbose:
            print(" ".join(cmd))
            if out.strip():
                print(out)
        if rc != 0:
            raise RuntimeError(f"libbqmoe build failed:\n{out}")
    rc, out, cmd = _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB])
    if rc != 0:
        raise RuntimeError(f"libbqmoe link failed:\n{out}")
    return LIB
