"""Build libdc.so (gfx950) in-tree with hipcc: every source compiled to an
object in parallel, then one link."""
import concurrent.futures
import glob
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libdc.so")

# -ffp-contract=off: a pre-divided contribution must be rounded before it is
#   added, so no multiply-add fusion.
# -fno-gpu-flush-denormals-to-zero: fp32 subnormals are kept.
# -fhip-fp32-correctly-rounded-divide-sqrt: x / c is correctly rounded.
# -packed-fp32-ops: no packed fp32 instructions.
COMPILE_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# the same flags for a one-command build of every source into a shared library
HIPCC_FLAGS = COMPILE_FLAGS[:4] + ["-shared"] + COMPILE_FLAGS[4:]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in ln)
    return r.returncode, out


def build(verbose: bool = False, extra=()) -> str:
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="libdc_") as tmp:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append(["hipcc"] + COMPILE_FLAGS + list(extra) + inc + ["-c", src, "-o", obj])
        workers = min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(workers) as pool:
            for cmd, (rc, out) in zip(cmds, pool.map(_run, cmds)):
                if verbose:
                    print(" ".join(cmd), flush=True)
                if rc != 0:
                    raise RuntimeError(f"hipcc failed:\n{out}")
                if verbose and out.strip():
                    print(out)
        link = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", SO] + objs
        rc, out = _run(link)
        if rc != 0:
            raise RuntimeError(f"hipcc link failed:\n{out}")
    return SO


if __name__ == "__main__":
    build(verbose=True)
