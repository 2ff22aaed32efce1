"""Pins for the oracle's fixed-sign 32-point block-Hadamard rotation.

The FP4-training article (hzrcw.cc, section 02) applies a fixed, deterministic
orthogonal (Hadamard) rotation on the weight-gradient path instead of random
ones.  The oracle computes y = c * H32 * diag(s) * x in fp32 with butterfly
stages h = 1, 2, 4, 8, 16 and c = RN32(1/sqrt 32).  Pins here:
  * c is the float nearest to 1/sqrt(32) (high-precision decimal), 0x3E3504F3;
  * the oracle's columns equal the Sylvester matrix built from popcount parity
    times the sign diagonal, and (H D)(H D)^T = 32 I in integers;
  * on integer inputs whose partial sums are exact in fp32, y equals
    RN32(c * (H D x)) computed by an explicit integer matrix product;
  * on general inputs, |y - (H D x)/sqrt 32| stays within 8 * 2^-24 * c * sum|x|;
  * subnormal inputs survive (no flush to zero);
  * sign mask m on x equals mask 0 on diag(s) x, bit for bit;
  * worked examples W8 / W9 and the transposed layout of the rotate-quantize call;
  * the fp32 stage order: hand-derived outputs (W11) of inputs on which running
    any stage 2^b before a stage 2^a < 2^b rounds differently.
"""
import decimal
import json
import os

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def sylvester32():
    i = np.arange(32)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def signs(mask):
    return np.array([-1 if (mask >> i) & 1 else 1 for i in range(32)], dtype=np.int64)


def test_constant_is_nearest_float(orc):
    c = np.float32(orc.hadamard_c())
    assert c.view(np.uint32) == 0x3E3504F3
    decimal.getcontext().prec = 60
    exact = decimal.Decimal(1) / decimal.Decimal(32).sqrt()
    cd = decimal.Decimal(float(c))
    for nb in (np.nextafter(c, np.float32(0)), np.nextafter(c, np.float32(1))):
        assert abs(cd - exact) < abs(decimal.Decimal(float(nb)) - exact)


@pytest.mark.parametrize("mask", [0, 0x9E3779B9, 0xFFFFFFFF, 1])
def test_matrix_is_sylvester_times_signs(orc, mask):
    c = np.float32(orc.hadamard_c())
    cols = []
    for j in range(32):
        e = np.zeros(32, dtype=np.float32)
        e[j] = 1
        y = orc.hadamard32_f32(e, mask)
        assert np.all(np.abs(y) == c)  # butterflies on a unit vector are exact
        cols.append(np.round(y / c).astype(np.int64))
    M = np.stack(cols, axis=1)
    HD = sylvester32() * signs(mask)[None, :]
    np.testing.assert_array_equal(M, HD)
    np.testing.assert_array_equal(M @ M.T, 32 * np.eye(32, dtype=np.int64))


@pytest.mark.parametrize("mask", [0, 0x9E3779B9])
def test_exact_on_small_integers(orc, mask):
    rng = np.random.default_rng(7)
    c = np.float32(orc.hadamard_c())
    HD = sylvester32() * signs(mask)[None, :]
    for _ in range(200):
        x = rng.integers(-1000, 1000, 32)
        y = orc.hadamard32_f32(x.astype(np.float32), mask)
        want = (HD @ x).astype(np.float32) * c  # numpy float32 multiply: one rounding
        np.testing.assert_array_equal(y, want)


@pytest.mark.parametrize("mask", [0, 0x9E3779B9])
def test_error_bound_general(orc, mask):
    rng = np.random.default_rng(11)
    HD = (sylvester32() * signs(mask)[None, :]).astype(np.float64)
    c = float(np.float32(orc.hadamard_c()))
    for scale in (1e-3, 1.0, 1e30, 1e-30):
        for _ in range(100):
            x = (rng.standard_t(3, 32) * scale).astype(np.float32)
            y = orc.hadamard32_f32(x, mask).astype(np.float64)
            exact = HD @ x.astype(np.float64) / np.sqrt(32.0)
            bound = 8 * 2.0 ** -24 * c * np.abs(x.astype(np.float64)).sum()
            assert np.all(np.abs(y - exact) <= bound)


def test_subnormals_kept(orc):
    tiny = np.float32(2.0 ** -140)
    x = np.zeros(32, dtype=np.float32)
    x[0] = tiny
    x[1] = tiny
    y = orc.hadamard32_f32(x, 0)
    c = np.float32(orc.hadamard_c())
    # outputs are (x0 + x1) for even i and (x0 - x1) = 0 for odd i, times c
    np.testing.assert_array_equal(y[0::2], np.full(16, np.float32(2 * tiny) * c, dtype=np.float32))
    assert np.all(y[0::2] != 0)
    assert not np.any(y[1::2])


def test_sign_mask_equals_flipped_input(orc):
    rng = np.random.default_rng(3)
    for mask in (0x9E3779B9, 0x12345678, 0xFFFFFFFF):
        x = rng.standard_normal(32).astype(np.float32)
        flipped = x * signs(mask).astype(np.float32)
        np.testing.assert_array_equal(orc.hadamard32_f32(x, mask), orc.hadamard32_f32(flipped, 0))


def test_orthogonality_inner_product(orc):
    rng = np.random.default_rng(5)
    for _ in range(50):
        x = rng.standard_normal(32).astype(np.float32)
        z = rng.standard_normal(32).astype(np.float32)
        hx = orc.hadamard32_f32(x, 0x9E3779B9).astype(np.float64)
        hz = orc.hadamard32_f32(z, 0x9E3779B9).astype(np.float64)
        lhs = hx @ hz
        rhs = x.astype(np.float64) @ z.astype(np.float64)
        scale = np.abs(x).sum() * np.abs(z).sum() / 32
        assert abs(lhs - rhs) <= 1e-6 * scale


def _golden_h():
    with open(GOLDEN) as f:
        return json.load(f)["hadamard"]


@pytest.mark.parametrize("case", _golden_h(), ids=lambda c: c["id"])
def test_worked_examples_hadamard(orc, case):
    x = np.zeros((32, 3), dtype=np.uint16)
    if "bf16_first_column" in case:
        x[0, :] = int(case["bf16_first_column"][0], 16)
    else:
        x[:, :] = int(case["bf16_all"], 16)
    codes, scales = orc.hadamard32_quantize(x, case["fmt"], case["mask"])
    assert np.all(scales == int(case["scale"], 16))
    if "codes_all" in case:
        assert np.all(codes == int(case["codes_all"], 16))
    if "packed_all" in case:
        assert np.all(codes == int(case["packed_all"], 16))
    if "codes_first" in case:
        assert np.all(codes[:, 0] == int(case["codes_first"][0], 16))
        assert not codes[:, 1:].any()


def _golden_order():
    with open(GOLDEN) as f:
        return json.load(f)["hadamard_order"]


@pytest.mark.parametrize("case", _golden_order(), ids=lambda c: c["id"])
def test_worked_examples_stage_order(orc, case):
    """W11: every output's fp32 bits, as derived by hand for stages 1, 2, 4, 8, 16 ascending"""
    x = np.zeros(32, dtype=np.uint32)
    for i, h in case["x_f32"].items():
        x[int(i)] = int(h, 16)
    y = orc.hadamard32_f32(x.view(np.float32), case["mask"]).view(np.uint32)
    a, b = case["a"], case["b"]
    want = [int(case["y_by_bits"]["%d%d" % ((i >> a) & 1, (i >> b) & 1)], 16) for i in range(32)]
    assert [int(v) for v in y] == want


def test_stage_order_cases_cover_every_pair():
    pairs = {(c["a"], c["b"]) for c in _golden_order()}
    assert pairs == {(a, b) for a in range(5) for b in range(a + 1, 5)}


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_rotate_quantize_layout(orc, fmt):
    """the transposed call equals: gather a column block, rotate, quantize as a row"""
    cfg = workloads.config(3)
    x = workloads.draw_tensor(cfg, "dY", rows=(0, 256))[:, :48]
    mask = 0x9E3779B9
    codes, scales = orc.hadamard32_quantize(x, fmt, mask)
    xf = workloads.bf16_bits_to_f32(x)
    rows, cols = x.shape
    rot = np.empty((cols, rows), dtype=np.float64)
    for c in range(cols):
        for b in range(rows // 32):
            rot[c, 32 * b:32 * b + 32] = orc.hadamard32_f32(xf[32 * b:32 * b + 32, c], mask)
    c2, s2 = orc.quantize_f64(rot, fmt)
    np.testing.assert_array_equal(codes, c2)
    np.testing.assert_array_equal(scales, s2)
