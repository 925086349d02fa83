"""Build the synthetic-input generators: host C (gcc) and device HIP (hipcc, gfx950)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(HERE, "libsynth_host.so")
DEV_SO = os.path.join(HERE, "libsynth_dev.so")


def build(verbose: bool = False) -> None:
    cmds = [
        ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", HOST_SO,
         os.path.join(HERE, "gen_host.c")],
        ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", DEV_SO, os.path.join(HERE, "gen_dev.hip")],
    ]
    for c in cmds:
        if verbose:
            print(" ".join(c), flush=True)
        subprocess.run(c, check=True, stderr=None if verbose else subprocess.DEVNULL)


if __name__ == "__main__":
    build(verbose=True)
