"""Build the host and GPU synthetic-input generators in place."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> None:
    cmds = [
        ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11",
         os.path.join(HERE, "gen.c"), "-o", os.path.join(HERE, "libbqsynth.so"), "-lm"],
        ["hipcc", *HIP_FLAGS, os.path.join(HERE, "gen_fill.hip"), "-o", os.path.join(HERE, "libbqsynth_gpu.so")],
    ]
    for c in cmds:
        if verbose:
            print(" ".join(c))
        r = subprocess.run(c, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"synth build failed: {' '.join(c)}\n{r.stdout}")
