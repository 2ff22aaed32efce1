"""Pins for the oracle's element formats, E8M0 scales and block quantizer.

Each check ties the oracle to something other than itself:
  * worked examples derived by hand (tests/golden/worked_examples.json);
  * E8M0 scale = floor(log2 amax) - emax, with floor(log2 amax) read off the
    bf16 bit fields (exponent field, or the highest set mantissa bit of a
    subnormal), over every bf16 amax;
  * E4M3 / E5M2 element casts against torch's float8 casts (round to nearest
    even) of the clamped, exactly scaled value, over every finite bf16 value
    and every scale exponent;
  * E2M1 casts against brute force (nearest of the 8 magnitudes, ties to the
    even code);
  * decode tables against torch's float8 -> float32 widening;
  * idempotence Q(DQ(Q(x))) = Q(x) and the half-spacing error bound.
"""
import json
import os

import numpy as np
import pytest
import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
FMTS = ("e4m3", "e5m2", "e2m1")
EMAX = {"e4m3": 8, "e5m2": 15, "e2m1": 2}
MAXN = {"e4m3": 448.0, "e5m2": 57344.0, "e2m1": 6.0}


def all_finite_bf16_values():
    bits = np.arange(65536, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite].astype(np.uint16)
    return bits, workloads.bf16_bits_to_f32(bits).astype(np.float64)


def _block(bf16_hex, n=32):
    x = np.zeros((1, n), dtype=np.uint16)
    for i, h in enumerate(bf16_hex):
        x[0, i] = int(h, 16)
    return x


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["quantize"], ids=lambda c: c["id"])
def test_worked_examples_quantize(orc, case):
    x = _block(case["bf16"])
    codes, scales = orc.quantize(x, case["fmt"])
    assert scales[0, 0] == int(case["scale"], 16)
    if case["fmt"] == "e2m1":
        want = [int(c, 16) for c in case["codes"]] + [0] * (32 - len(case["codes"]))
        got = [(codes[0, j // 2] >> (4 * (j & 1))) & 0xF for j in range(32)]
        assert got == want
        if "packed" in case:
            packed = [int(c, 16) for c in case["packed"]]
            assert list(codes[0, :len(packed)]) == packed
            assert not codes[0, len(packed):].any()
    else:
        want = [int(c, 16) for c in case["codes"]] + [0] * (32 - len(case["codes"]))
        assert list(codes[0]) == want


def _floor_log2_from_bf16_fields(b):
    """floor(log2 v) of a positive finite bf16 pattern from its fields: a normal
    number (exponent field E >= 1) lies in [2^(E-127), 2^(E-126)); a subnormal
    m * 2^-133 (E = 0) lies in [2^(L-1-133), 2^(L-133)) with L the bit length of m"""
    E, m = (b >> 7) & 0xFF, b & 0x7F
    return E - 127 if E else m.bit_length() - 1 - 133


def test_e8m0_exhaustive_from_bf16_fields(orc):
    """every non-negative finite bf16 amax: S = clamp(floor(log2 amax) - emax, -127, 127) + 127"""
    bits = np.arange(0x7F80, dtype=np.uint16)  # sign 0, exponent < 0xFF
    amax = workloads.bf16_bits_to_f32(bits).astype(np.float64)
    for fmt in FMTS:
        want = np.empty(amax.size, dtype=np.uint8)
        for i, b in enumerate(bits):
            e = -127 if b == 0 else _floor_log2_from_bf16_fields(int(b)) - EMAX[fmt]
            want[i] = min(max(e, -127), 127) + 127
        np.testing.assert_array_equal(orc.e8m0(amax, fmt), want)


def test_e8m0_upper_range(orc):
    # the largest bf16 (about 2^128) gives e = 127 - emax; E8M0 never reaches 0xFF from finite data
    big = float(workloads.bf16_bits_to_f32(np.array([0x7F7F], dtype=np.uint16))[0])
    for fmt in FMTS:
        assert orc.e8m0(np.array([big]), fmt)[0] == 127 - EMAX[fmt] + 127
    # doubles beyond bf16 range clamp at +127
    assert orc.e8m0(np.array([2.0 ** 300]), "e2m1")[0] == 254


@pytest.mark.parametrize("fmt,tdtype", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
@pytest.mark.slow
def test_fp8_cast_exhaustive_against_torch(orc, fmt, tdtype):
    """every finite bf16 v and every e in [-127, 127]: code of v * 2^-e"""
    _, v = all_finite_bf16_values()
    for e in range(-127, 128):
        got = orc.cast(v, np.full(v.size, e, dtype=np.int32), fmt)
        q = np.clip(np.ldexp(v, -e), -MAXN[fmt], MAXN[fmt])
        want = torch.from_numpy(q.astype(np.float32)).to(tdtype).view(torch.uint8).numpy()
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (fmt, e, v[bad[:5]], got[bad[:5]], want[bad[:5]])


def _e2m1_brute(q):
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    a = np.minimum(np.abs(q), 6.0)
    d = np.abs(a[:, None] - grid[None, :])
    is_min = d == d.min(axis=1, keepdims=True)
    even = (np.arange(8) % 2 == 0)[None, :]
    two = is_min.sum(axis=1) == 2
    pick = np.where(two, np.argmax(is_min & even, axis=1), np.argmax(is_min, axis=1))
    return (pick | (np.signbit(q).astype(np.int64) << 3)).astype(np.uint8)


@pytest.mark.slow
def test_e2m1_cast_exhaustive_brute_force(orc):
    _, v = all_finite_bf16_values()
    for e in range(-127, 128):
        got = orc.cast(v, np.full(v.size, e, dtype=np.int32), "e2m1")
        want = _e2m1_brute(np.ldexp(v, -e))
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (e, v[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e2m1_tie_cases(orc):
    q = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, 7.9, -100.0, -0.0])
    want = [0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0x6, 0x8, 0x7, 0xF, 0x8]
    assert list(orc.cast(q, np.zeros(q.size, dtype=np.int32), "e2m1")) == want


@pytest.mark.parametrize("fmt,tdtype", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_decode_table_against_torch(orc, fmt, tdtype):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.decode(codes, fmt)
    want = torch.from_numpy(codes).view(tdtype).to(torch.float32).numpy().astype(np.float64)
    fin = np.isfinite(want)
    np.testing.assert_array_equal(got[fin], want[fin])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got), np.isinf(want))


def test_decode_table_e2m1(orc):
    got = orc.decode(np.arange(16, dtype=np.uint8), "e2m1")
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(got[:8]) == mags
    assert list(got[8:]) == [-m for m in mags]
    assert np.signbit(got[8])


def _edge_suite():
    """blocks exercising zero, subnormal, tie, saturation, sign and range edges"""
    rng = np.random.default_rng(1234)
    rows = []
    rows.append(np.zeros(32, dtype=np.uint16))                             # all zero
    rows.append(np.full(32, 0x8000, dtype=np.uint16))                      # all -0
    rows.append(rng.integers(0, 0x80, 32).astype(np.uint16))               # bf16 subnormals
    rows.append((rng.integers(0, 0x80, 32) | 0x8000).astype(np.uint16))   # negative subnormals
    rows.append(np.full(32, 0x7F7F, dtype=np.uint16))                      # largest bf16
    t = np.zeros(32, dtype=np.uint16); t[0] = 0x7F7F; t[1:] = 0x0001       # huge with tiny
    rows.append(t)
    rows.append(rng.integers(0, 0x7F80, 32).astype(np.uint16))             # any exponent
    rows.append(rng.integers(0x3F00, 0x4100, 32).astype(np.uint16))        # near 1: many ties
    for r in rng.integers(0, 65536, (8, 32)):                              # random finite patterns
        r = r.astype(np.uint16)
        r[((r >> 7) & 0xFF) == 0xFF] = 0x3F80
        rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("fmt", FMTS)
def test_idempotence_and_error_bound(orc, fmt):
    cfg = workloads.config(0)
    x = np.concatenate([workloads.draw_tensor(cfg, "A")[:, :64], _edge_suite()[:, :32].repeat(2, axis=1)])
    codes, scales = orc.quantize(x, fmt)
    deq = orc.dequantize(codes, scales, fmt)
    codes2, scales2 = orc.quantize_f64(deq, fmt)
    np.testing.assert_array_equal(scales2, scales)
    np.testing.assert_array_equal(codes2, codes)
    # |DQ(Q(v)) - v| <= half the format spacing at v, unless v saturated
    v = workloads.bf16_bits_to_f32(x).astype(np.float64)
    e = scales.astype(np.int64).repeat(32, axis=1) - 127
    q = np.ldexp(v, -e)
    mant = {"e4m3": 3, "e5m2": 2, "e2m1": 1}[fmt]
    emin = {"e4m3": -6, "e5m2": -14, "e2m1": 0}[fmt]
    aq = np.abs(q)
    k = np.where(aq > 0, np.floor(np.log2(np.where(aq > 0, aq, 1.0))), emin)
    half = np.ldexp(0.5, (np.maximum(k, emin) - mant).astype(np.int64))
    ok = np.abs(np.ldexp(deq, -e) - q) <= half
    sat = aq >= MAXN[fmt]
    assert np.all(ok | sat)
    assert np.all(np.abs(np.ldexp(deq, -e)[sat]) == MAXN[fmt])


def test_non_finite_block(orc):
    for bad in (0x7F80, 0xFF80, 0x7FC0):
        x = np.full((1, 64), 0x3F80, dtype=np.uint16)
        x[0, 5] = bad
        for fmt in FMTS:
            codes, scales = orc.quantize(x, fmt)
            assert scales[0, 0] == 0xFF and scales[0, 1] == 0x77 - (EMAX[fmt] - 8)
            nb = 16 if fmt == "e2m1" else 32
            assert not codes[0, :nb].any()


def test_transpose_mode_is_row_mode_of_transpose(orc):
    cfg = workloads.config(0)
    b = workloads.draw_tensor(cfg, "B")
    for fmt in FMTS:
        ct, st = orc.quantize_transpose(b, fmt)
        cr, sr = orc.quantize(np.ascontiguousarray(b.T), fmt)
        np.testing.assert_array_equal(ct, cr)
        np.testing.assert_array_equal(st, sr)
