"""Pins for the oracle's MX GEMM, C[m, n] = sum_k A[m, k] B[n, k].

The MX products are exact, so the GEMM has a plain definition.  Pins:
  * worked examples W10 (closed forms);
  * brute force in exact rational arithmetic (fractions) on tiny operands of
    every format pair;
  * lossless operands: bf16 inputs that already sit on the MX grid give
    C = X W^T of the raw inputs, independent of the quantizer;
  * the weight-gradient identity dY^T X = (H dY)^T (H X) for the orthogonal
    block rotation, evaluated on the oracle's own rotated values;
  * S_abs is the same sum on absolute values and bounds |C|.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
FMTS = ("e4m3", "e5m2", "e2m1")


def _golden_g():
    with open(GOLDEN) as f:
        return json.load(f)["gemm"]


def _bf16(values):
    import torch
    return torch.tensor(values, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("case", _golden_g(), ids=lambda c: c["id"])
def test_worked_examples_gemm(orc, case):
    K = case["K"]
    a = _bf16(np.full((1, K), case["a_value"], dtype=np.float32))
    b = _bf16(np.full((1, K), case["b_value"], dtype=np.float32))
    ca, sa = orc.quantize(a, case["fa"])
    cb, sb = orc.quantize(b, case["fb"])
    if "a_scale" in case:
        assert sa[0, 0] == int(case["a_scale"], 16) and sb[0, 0] == int(case["b_scale"], 16)
        assert ca[0, 0] & 0xF == int(case["a_code"], 16) and cb[0, 0] & 0xF == int(case["b_code"], 16)
    C, S = orc.gemm(ca, sa, case["fa"], cb, sb, case["fb"])
    assert C[0, 0] == case["C"]
    assert S[0, 0] == abs(case["C"])


def _exact_value(code, scale, fmt):
    """exact rational value of one element, from the bit fields"""
    eb, mb, bias = {"e4m3": (4, 3, 7), "e5m2": (5, 2, 15), "e2m1": (2, 1, 1)}[fmt]
    s = (code >> (eb + mb)) & 1
    E = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    if E == 0:
        v = Fraction(m, 1 << mb) * Fraction(2) ** (1 - bias)
    else:
        v = (1 + Fraction(m, 1 << mb)) * Fraction(2) ** (E - bias)
    v *= Fraction(2) ** (int(scale) - 127)
    return -v if s else v


def _elements(codes, fmt, K):
    if fmt == "e2m1":
        return [[(int(row[k // 2]) >> (4 * (k & 1))) & 0xF for k in range(K)] for row in codes]
    return [[int(v) for v in row[:K]] for row in codes]


@pytest.mark.parametrize("fa", FMTS)
@pytest.mark.parametrize("fb", FMTS)
def test_brute_force_exact(orc, fa, fb):
    rng = np.random.default_rng(10 * FMTS.index(fa) + FMTS.index(fb))
    M, N, K = 3, 4, 96
    # wide exponent spread per block, heavy tails, a zero block
    a = _bf16((rng.standard_t(3, (M, K)) * np.exp2(rng.integers(-20, 20, (M, 1)))).astype(np.float32))
    b = _bf16((rng.standard_normal((N, K)) * np.exp2(rng.integers(-30, 30, (N, K // 32)).repeat(32, 1))).astype(np.float32))
    b[1, 32:64] = 0
    ca, sa = orc.quantize(a, fa)
    cb, sb = orc.quantize(b, fb)
    C, S = orc.gemm(ca, sa, fa, cb, sb, fb)
    ea, eb = _elements(ca, fa, K), _elements(cb, fb, K)
    for m in range(M):
        for n in range(N):
            exact = sum(_exact_value(ea[m][k], sa[m, k // 32], fa) * _exact_value(eb[n][k], sb[n, k // 32], fb)
                        for k in range(K))
            sabs = sum(abs(_exact_value(ea[m][k], sa[m, k // 32], fa) * _exact_value(eb[n][k], sb[n, k // 32], fb))
                       for k in range(K))
            assert abs(Fraction(C[m, n]) - exact) <= Fraction(1, 2 ** 50) * sabs
            assert abs(Fraction(S[m, n]) - sabs) <= Fraction(1, 2 ** 50) * sabs


def _on_grid_block(rng, fmt, n_rows, K):
    """bf16 values whose MX quantization is lossless: format grid points times
    2^e per block, each block holding one element of the top binade"""
    mags = {"e2m1": [0, 0.5, 1, 1.5, 2, 3, 4, 6],
            "e4m3": [m * 2.0 ** k for k in range(-2, 3) for m in (1, 1.25, 1.5, 1.75)],
            "e5m2": [m * 2.0 ** k for k in range(-2, 3) for m in (1, 1.25, 1.5, 1.75)]}[fmt]
    top = {"e2m1": [4, 6], "e4m3": [4, 6, 7], "e5m2": [4, 5, 6, 7]}[fmt]
    v = rng.choice(mags, (n_rows, K)) * rng.choice([-1, 1], (n_rows, K))
    v[:, ::32] = rng.choice(top, (n_rows, K // 32))
    # exponent spread small enough that float64 sums of the products are exact
    v *= np.exp2(rng.integers(-4, 5, (n_rows, K // 32))).repeat(32, axis=1)
    return v.astype(np.float32)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e2m1", "e2m1")])
def test_lossless_operands_give_exact_product(orc, fa, fb):
    rng = np.random.default_rng(21)
    M, N, K = 16, 24, 256
    x = _on_grid_block(rng, fa, M, K)
    w = _on_grid_block(rng, fb, N, K)
    xb, wb = _bf16(x), _bf16(w)
    assert np.array_equal(workloads.bf16_bits_to_f32(xb), x)  # inputs exact in bf16
    ca, sa = orc.quantize(xb, fa)
    cb, sb = orc.quantize(wb, fb)
    np.testing.assert_array_equal(orc.dequantize(ca, sa, fa), x)
    np.testing.assert_array_equal(orc.dequantize(cb, sb, fb), w)
    C, _ = orc.gemm(ca, sa, fa, cb, sb, fb)
    want = x.astype(np.float64) @ w.astype(np.float64).T
    np.testing.assert_array_equal(C, want)


def test_rows_subset(orc):
    cfg = workloads.config(0)
    a = workloads.draw_tensor(cfg, "A")
    b = workloads.draw_tensor(cfg, "B")
    ca, sa = orc.quantize(a, "e4m3")
    cb, sb = orc.quantize_transpose(b, "e4m3")
    C, S = orc.gemm(ca, sa, "e4m3", cb, sb, "e4m3")
    rows = [0, 7, 100, 255]
    C2, S2 = orc.gemm(ca, sa, "e4m3", cb, sb, "e4m3", rows=rows)
    np.testing.assert_array_equal(C[rows], C2)
    np.testing.assert_array_equal(S[rows], S2)
    assert np.all(np.abs(C) <= S)


def test_wgrad_rotation_invariance(orc):
    """dY^T X equals (H dY)^T (H X) when both are rotated along tokens by the
    same orthogonal blocks; checked on the oracle's fp32 rotations"""
    rng = np.random.default_rng(9)
    T, n, k = 64, 5, 6
    dy = rng.standard_normal((T, n)).astype(np.float32)
    x = rng.standard_normal((T, k)).astype(np.float32)
    mask = 0x9E3779B9

    def rot(a):
        out = np.empty_like(a)
        for c in range(a.shape[1]):
            for b in range(T // 32):
                out[32 * b:32 * b + 32, c] = orc.hadamard32_f32(a[32 * b:32 * b + 32, c], mask)
        return out.astype(np.float64)

    lhs = rot(dy).T @ rot(x)
    rhs = dy.astype(np.float64).T @ x.astype(np.float64)
    bound = 1e-5 * (np.abs(dy).T.astype(np.float64) @ np.abs(x).astype(np.float64))
    assert np.all(np.abs(lhs - rhs) <= bound)
