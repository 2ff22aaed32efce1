"""CPU build of the HIP path's element conversion, checked exhaustively against the oracle.

The kernels' conversion functions (mx_convert.h) are plain integer / fp32 code
shared by host and device compilation.  Built here with g++ (no GPU), they must
give the oracle's codes and scales for every finite bf16 value and every scale
exponent, and for a large set of fp32 values (the rotation path's input),
including ties, subnormals and values on both sides of every binade edge.
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
    for name in ("shim_code_from_bf16", "shim_code_from_f32"):
        getattr(L, name).argtypes = [P, P, i64, i32, P]
    for name in ("shim_scale_exp_bf16", "shim_scale_exp_f32"):
        getattr(L, name).argtypes = [P, i64, i32, P]
    return L


def _finite_bf16():
    bits = np.arange(65536, dtype=np.uint32)
    return bits[((bits >> 7) & 0xFF) != 0xFF].astype(np.uint16)


@pytest.mark.parametrize("fi,fmt", list(enumerate(FMTS)))
def test_code_from_bf16_exhaustive(shim, orc, fi, fmt):
    b = _finite_bf16()
    v = workloads.bf16_bits_to_f32(b).astype(np.float64)
    out = np.empty(b.size, dtype=np.uint8)
    for e in range(-127, 128):
        ev = np.full(b.size, e, dtype=np.int32)
        shim.shim_code_from_bf16(b.ctypes.data, ev.ctypes.data, b.size, fi, out.ctypes.data)
        want = orc.cast(v, ev, fmt)
        bad = np.nonzero(out != want)[0]
        assert bad.size == 0, (fmt, e, hex(int(b[bad[0]])), out[bad[0]], want[bad[0]])


def _f32_cases(rng):
    parts = [rng.integers(0, 2 ** 32, 3_000_000, dtype=np.uint64).astype(np.uint32)]
    # values near every target rounding point: k * 2^j +- a few ulps, both signs
    mids = np.arange(1, 64, dtype=np.float64) / 16.0
    pts = (mids[None, :] * np.exp2(np.arange(-150, 122))[:, None]).ravel().astype(np.float32)
    pu = pts.view(np.uint32)
    for d in (-2, -1, 0, 1, 2):
        parts.append(pu + np.uint32(d & 0xFFFFFFFF) if d >= 0 else pu - np.uint32(-d))
    parts.append(np.arange(0, 1 << 16, dtype=np.uint32))            # fp32 subnormals
    u = np.concatenate(parts)
    u = np.concatenate([u, u | np.uint32(0x80000000)])
    u = u[((u >> 23) & 0xFF) != 0xFF]                                # finite only
    return u.view(np.float32)


@pytest.mark.parametrize("fi,fmt", list(enumerate(FMTS)))
def test_code_from_f32_sampled(shim, orc, fi, fmt):
    rng = np.random.default_rng(17)
    y = _f32_cases(rng)
    out = np.empty(y.size, dtype=np.uint8)
    for e in (-127, -126, -100, -30, -12, -8, -5, -2, 0, 3, 13, 60, 100, 125):
        ev = np.full(y.size, e, dtype=np.int32)
        shim.shim_code_from_f32(y.ctypes.data, ev.ctypes.data, y.size, fi, out.ctypes.data)
        want = orc.cast(y.astype(np.float64), ev, fmt)
        bad = np.nonzero(out != want)[0]
        assert bad.size == 0, (fmt, e, y[bad[:3]], out[bad[:3]], want[bad[:3]])


@pytest.mark.parametrize("fi,fmt", list(enumerate(FMTS)))
def test_code_from_f32_block_consistent_e(shim, orc, fi, fmt):
    """y drawn with e taken as the scale of a block containing y (the kernels' use)"""
    rng = np.random.default_rng(23)
    y = (rng.standard_t(3, 2_000_000) * np.exp2(rng.integers(-140, 120, 2_000_000))).astype(np.float32)
    a = np.abs(y.astype(np.float64)) * np.exp2(rng.integers(0, 12, y.size))  # block amax >= |y|
    a = np.minimum(a, 3.0e38)
    e = orc.e8m0(a, fmt).astype(np.int32) - 127
    out = np.empty(y.size, dtype=np.uint8)
    shim.shim_code_from_f32(y.ctypes.data, e.ctypes.data, y.size, fi, out.ctypes.data)
    np.testing.assert_array_equal(out, orc.cast(y.astype(np.float64), e, fmt))


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
