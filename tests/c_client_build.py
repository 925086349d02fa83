"""Build tests/libc_client.so: the plain C11 client of libdc.so (gcc, no
hipcc), linked against the in-tree libdc.so and the HIP runtime."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libc_client.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_client.c"), "-o", SO,
           "-L", os.path.join(ROOT, "gradient_reduction_amd"), "-l:libdc.so",
           "-Wl,-rpath,$ORIGIN/../gradient_reduction_amd",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed:\n" + r.stdout)
    return SO


if __name__ == "__main__":
    print(build())
