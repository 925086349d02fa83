"""Build libdc.so (gfx950) in-tree with hipcc."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libdc.so")

# -ffp-contract=off: a pre-divided contribution must be rounded before it is
#   added, so no multiply-add fusion.
# -fno-gpu-flush-denormals-to-zero: fp32 subnormals are kept.
# -fhip-fp32-correctly-rounded-divide-sqrt: x / c is correctly rounded.
# -packed-fp32-ops: no packed fp32 instructions.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False, extra=()) -> str:
    cmd = (["hipcc"] + HIPCC_FLAGS + list(extra) + ["-I", os.path.join(ROOT, "include"),
           "-o", SO] + sources())
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{out}")
    if verbose and out.strip():
        print(out)
    return SO


if __name__ == "__main__":
    build(verbose=True)
