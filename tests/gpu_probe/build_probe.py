"""Build the test-only matrix-instruction probes (mfma_probe.hip) into libmfma_probe.so.

Not part of libmx; only tests/test_gpu_mfma_probe.py loads it."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfma_probe.hip")
LIB = os.path.join(HERE, "libmfma_probe.so")


def build() -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
                    "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
