"""Build the plain C client of libmx (mx_c_client.c, gcc, C99) against
include/mx.h and the in-tree libmx.so.  Not part of libmx; only
tests/test_gpu_c_client.py runs it."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "mx_c_client.c")
EXE = os.path.join(HERE, "mx_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    libdir = os.path.join(ROOT, "precision_block_amax_amd")
    tmp = EXE + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"), SRC, "-o", tmp,
                    "-L" + libdir, "-lmx", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath,$ORIGIN/../../precision_block_amax_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
