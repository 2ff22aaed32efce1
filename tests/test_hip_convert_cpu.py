"""CPU build of the kernels' E8M0 scale-exponent functions, checked against the oracle.

The quantizers take each block's scale exponent from the bits of its amax with
scale_exp_bf16 (row and transposed modes) and scale_exp_f32 (the rotated mode,
whose amax is an fp32 value).  Both are plain integer code in mx_convert.h,
shared by host and device compilation.  Built here with g++ (no GPU), they must
give the oracle's scale for every non-negative finite bf16 amax and for a large
set of fp32 amax values, subnormals included.  The element casts are gfx950
conversion instructions; the GPU parity tests cover them (every finite bf16
value at every reachable scale, through both quantizers).
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "precision_block_amax_amd", "csrc")
FMTS = ("e4m3", "e5m2", "e2m1")


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("shim") / "libconvert_shim.so")
    subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-shared", "-fPIC", "-I", CSRC,
                    os.path.join(HERE, "cpu_build", "convert_shim.cpp"), "-o", out], check=True)
    L = ctypes.CDLL(out)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    for name in ("shim_scale_exp_bf16", "shim_scale_exp_f32"):
        getattr(L, name).argtypes = [P, i64, i32, P]
    return L


@pytest.mark.parametrize("fi,fmt", list(enumerate(FMTS)))
def test_scale_exponents(shim, orc, fi, fmt):
    b = np.arange(0x7F80, dtype=np.uint16)
    got = np.empty(b.size, dtype=np.int32)
    shim.shim_scale_exp_bf16(b.ctypes.data, b.size, fi, got.ctypes.data)
    want = orc.e8m0(workloads.bf16_bits_to_f32(b).astype(np.float64), fmt).astype(np.int32) - 127
    np.testing.assert_array_equal(got, want)
    rng = np.random.default_rng(2)
    u = np.concatenate([rng.integers(0, 0x7F800000, 2_000_000, dtype=np.uint64).astype(np.uint32),
                        np.arange(0, 1 << 20, dtype=np.uint32)])
    got = np.empty(u.size, dtype=np.int32)
    shim.shim_scale_exp_f32(u.ctypes.data, u.size, fi, got.ctypes.data)
    want = orc.e8m0(u.view(np.float32).astype(np.float64), fmt).astype(np.int32) - 127
    np.testing.assert_array_equal(got, want)
