"""Why MX GEMMs with an FP8 operand run through the exact bf16 carrier.

The block-scaled matrix instruction of gfx950 (V_MFMA_SCALE_F32_32X32X64_F8F6F4)
would run MXFP8 at twice the bf16 rate, but with E4M3 operands it adds the
products of one 32-element block in a fixed-point window about 13 bits below
the largest product: a product 2^-13 below it survives, one 2^-14 below is
dropped.  On random E4M3 blocks one instruction then misses the exact sum by
well over the 1e-5 * sum|a*b| fp32-accumulation tolerance the library is held
to.  The same instruction on E2M1 operands, and the bf16 instruction the
carrier uses, sum exactly and round once.  Each case runs one instruction of a
test-only probe library (tests/gpu_probe) against the oracle's exact product;
the control cases fix the probe's operand and output layouts first, so a
failure of the window case cannot be a layout mistake."""
import ctypes
import os

import numpy as np
import pytest

import oracle
from helpers import to_dev_u8, to_host

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
TOL = 1e-5  # the GEMM tolerance: |err| <= TOL * sum |a*b|


@pytest.fixture(scope="module")
def probe():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sys
    sys.path.insert(0, os.path.join(HERE, "gpu_probe"))
    import build_probe
    if not os.path.exists(build_probe.LIB):
        build_probe.build()
    L = ctypes.CDLL(build_probe.LIB)
    P = ctypes.c_void_p
    for name in ("probe_mfma_scale_e4m3", "probe_mfma_scale_e2m1"):
        getattr(L, name).argtypes = [P, P, P, P, P]
    L.probe_mfma_bf16.argtypes = [P, P, P]
    return L


def run_scaled(probe, fmt, a, b, sa, sb):
    import torch
    c = torch.empty((32, 32), dtype=torch.float32, device="cuda")
    da, db, dsa, dsb = to_dev_u8(a), to_dev_u8(b), to_dev_u8(sa), to_dev_u8(sb)
    fn = probe.probe_mfma_scale_e4m3 if fmt == "e4m3" else probe.probe_mfma_scale_e2m1
    assert fn(da.data_ptr(), db.data_ptr(), dsa.data_ptr(), dsb.data_ptr(), c.data_ptr()) == 0
    return to_host(c).astype(np.float64)


def e4m3_codes(rng, shape, exp_lo=0, exp_hi=15):
    """random E4M3 codes with exponent field in [exp_lo, exp_hi], never the NaN code"""
    e = rng.integers(exp_lo, exp_hi + 1, shape)
    m = rng.integers(0, 8, shape)
    m = np.where(e == 15, np.minimum(m, 6), m)
    return ((rng.integers(0, 2, shape) << 7) | (e << 3) | m).astype(np.uint8)


def rel_err(c, C, S):
    return np.abs(c - C) / np.where(S > 0, S, 1.0)


def test_control_e4m3_narrow_products_are_exact(probe):
    """E4M3 values in [1, 4) and varied block scales: every product of a block lies
    within the window, so the instruction is exact -- and matches the oracle
    element by element only if the operand, scale and output layouts are right"""
    rng = np.random.default_rng(1)
    a, b = e4m3_codes(rng, (32, 64), 7, 8), e4m3_codes(rng, (32, 64), 7, 8)
    sa, sb = rng.integers(118, 137, (32, 2)).astype(np.uint8), rng.integers(118, 137, (32, 2)).astype(np.uint8)
    C, S = oracle.gemm(a, sa, "e4m3", b, sb, "e4m3")
    c = run_scaled(probe, "e4m3", a, b, sa, sb)
    assert np.all(rel_err(c, C, S) <= 2.0 ** -22), rel_err(c, C, S).max()


def test_scaled_e4m3_window_drops_small_products(probe):
    """a block holding the products 1 and 2^-k: k = 13 survives, k = 14 is dropped
    (an error of 2^-14 / (1 + 2^-14) = 6.1e-5 of sum |a*b|, six times the tolerance)"""
    def one(k):
        a = np.zeros((32, 64), dtype=np.uint8)
        b = np.zeros((32, 64), dtype=np.uint8)
        a[0, 0] = b[0, 0] = 0x38            # 1.0
        # 2^-k = 2^-6 * 2^-(k-6): E4M3 2^-6 is 0x08, 2^-7 is 0x04 (subnormal), 2^-8 0x02
        a[0, 1] = 0x08
        b[0, 1] = {13: 0x04, 14: 0x02}[k]
        s = np.full((32, 2), 127, dtype=np.uint8)
        C, S = oracle.gemm(a, s, "e4m3", b, s, "e4m3")
        assert C[0, 0] == 1.0 + 2.0 ** -k
        return run_scaled(probe, "e4m3", a, b, s, s)[0, 0], C[0, 0], S[0, 0]
    got13, want13, _ = one(13)
    assert got13 == want13                   # 1 + 2^-13 survives
    got14, want14, s14 = one(14)
    assert got14 == 1.0                      # 1 + 2^-14: the small product is gone
    assert abs(got14 - want14) > TOL * s14


def test_scaled_e4m3_random_blocks_miss_the_tolerance(probe):
    """random E4M3 codes over the whole exponent range, unit scales: one instruction's
    worst element misses the exact sum by more than the tolerance"""
    rng = np.random.default_rng(2)
    worst = 0.0
    for _ in range(8):
        a, b = e4m3_codes(rng, (32, 64)), e4m3_codes(rng, (32, 64))
        s = np.full((32, 2), 127, dtype=np.uint8)
        C, S = oracle.gemm(a, s, "e4m3", b, s, "e4m3")
        c = run_scaled(probe, "e4m3", a, b, s, s)
        worst = max(worst, float(rel_err(c, C, S).max()))
    print("scaled E4M3 instruction, worst |err| / sum|a*b| = %.3g" % worst)
    assert worst > TOL
    assert worst < 1e-2                      # not garbage: a window error, not a layout error


def test_scaled_e2m1_is_exact(probe):
    """E2M1 x E2M1 products span few binades: the same instruction sums a block
    exactly; over two blocks with different scales only the final fp32 rounding
    remains"""
    rng = np.random.default_rng(3)
    for _ in range(8):
        a = rng.integers(0, 256, (32, 32)).astype(np.uint8)
        b = rng.integers(0, 256, (32, 32)).astype(np.uint8)
        sa, sb = rng.integers(100, 150, (32, 2)).astype(np.uint8), rng.integers(100, 150, (32, 2)).astype(np.uint8)
        C, S = oracle.gemm(a, sa, "e2m1", b, sb, "e2m1")
        c = run_scaled(probe, "e2m1", a, b, sa, sb)
        assert np.all(rel_err(c, C, S) <= 2.0 ** -23), rel_err(c, C, S).max()


def test_bf16_instruction_sums_exactly_and_rounds_once(probe):
    import torch
    a = np.zeros((32, 16), dtype=np.uint16)
    b = np.zeros((32, 16), dtype=np.uint16)
    one, tiny = 0x3F80, 0x3380                    # 1.0 and 2^-24 as bf16
    # row 0: 1 + 2^-24 + 2^-24 + 2^-24 = 1 + 1.5 ulp(1): summed exactly and rounded once -> 1 + 2^-22
    # (adding one product at a time in fp32 would return 1)
    a[0, :4] = [one, tiny, tiny, tiny]
    b[0, :4] = one
    # row 1: 2^20 - 2^20 + 1 = 1 whatever the order inside the instruction
    a[1, :3] = [0x4980, 0xC980, one]              # 2^20, -2^20, 1
    b[1, :3] = one
    c = torch.empty((32, 32), dtype=torch.float32, device="cuda")
    da = torch.from_numpy(a.view(np.int16)).cuda()
    db = torch.from_numpy(b.view(np.int16)).cuda()
    assert probe.probe_mfma_bf16(da.data_ptr(), db.data_ptr(), c.data_ptr()) == 0
    h = to_host(c)
    assert h[0, 0] == np.float32(1.0 + 2.0 ** -22)
    assert h[1, 1] == 1.0
    # control: a random bf16 product within fp32 rounding of the exact one
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 16)).astype(np.float32)
    y = rng.standard_normal((32, 16)).astype(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    yb = torch.from_numpy(y).to(torch.bfloat16)
    dx, dy = xb.cuda(), yb.cuda()                 # kept alive until the probe has run
    assert probe.probe_mfma_bf16(dx.data_ptr(), dy.data_ptr(), c.data_ptr()) == 0
    X, Y = xb.to(torch.float64).numpy(), yb.to(torch.float64).numpy()
    C, S = X @ Y.T, np.abs(X) @ np.abs(Y).T
    assert np.all(rel_err(to_host(c).astype(np.float64), C, S) <= 2.0 ** -23)
