"""Pins for the oracle's stochastic rounding (the ablation's randomised cast).

Definition under test: with lo <= |q| < hi the neighbouring magnitudes of the
format grid, F = floor(2^32 (|q| - lo) / (hi - lo)); a 32-bit random word r
rounds up iff r < F; |q| >= max normal saturates; the block scale is the
round-to-nearest path's.  Random words: element i takes word i mod 4 of
Philox4x32-10 at counter (i / 4, 0, 0) under key (seed low, seed high).

Pins, none of which re-uses the oracle's arithmetic:
  * Philox4x32-10 against its published known-answer vectors
    (tests/golden/philox4x32_10_kat.json);
  * the cast against brute force in exact rational arithmetic: the format
    grid enumerated from the bit-field definitions, neighbours found by
    search, F computed with Fractions, and r probed at F - 1, F, F + 1;
  * grid values never move, whatever r;
  * unbiasedness: the mean of many draws converges to q;
  * the quantizer's scales equal the round-to-nearest quantizer's, and each
    code is the round-down or round-up neighbour.
"""
import bisect
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

KAT = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")
FMTS = ("e4m3", "e5m2", "e2m1")
MAXN = {"e4m3": 448, "e5m2": 57344, "e2m1": 6}
EMAX = {"e4m3": 8, "e5m2": 15, "e2m1": 2}


def grid(fmt):
    """non-negative magnitudes in code order, from the bit-field definitions
    (sign-magnitude codes are ordered like their values, so index = code)"""
    ebits, mbits, bias = {"e4m3": (4, 3, 7), "e5m2": (5, 2, 15), "e2m1": (2, 1, 1)}[fmt]
    out = []
    for E in range(1 << ebits):
        for m in range(1 << mbits):
            if E == 0:
                v = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
            else:
                v = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (E - bias)
            if v > MAXN[fmt]:
                break
            out.append(v)
    return out


GRID = {f: grid(f) for f in FMTS}
SIGN = {"e4m3": 0x80, "e5m2": 0x80, "e2m1": 0x8}


def brute_sr(v, e, r, fmt):
    """code of v * 2^-e under stochastic rounding with word r, exactly"""
    q = Fraction(v) * Fraction(2) ** (-e)
    a, g = abs(q), GRID[fmt]
    if a >= MAXN[fmt]:
        idx = len(g) - 1
    else:
        i = bisect.bisect_right(g, a) - 1  # g[i] <= a < g[i + 1]
        lo, hi = g[i], g[i + 1]
        F = ((a - lo) / (hi - lo) * 2 ** 32).__floor__()
        idx = i + 1 if r < F else i
    neg = v < 0 or (v == 0 and np.signbit(v))
    return idx | (SIGN[fmt] if neg else 0), (None if a >= MAXN[fmt] else F)


def test_philox_known_answers():
    with open(KAT) as f:
        vec = json.load(f)["vectors"]
    for t in vec:
        ctr = [int(w, 16) for w in t["ctr"]]
        key = [int(w, 16) for w in t["key"]]
        assert [int(w) for w in oracle.philox4x32_10(ctr, key)] == [int(w, 16) for w in t["out"]]


def test_sr_words_layout():
    """element i takes word i mod 4 of the block at counter i / 4"""
    seed = 0x0123456789ABCDEF
    w = oracle.sr_words(seed, 16)
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for blk in range(4):
        assert list(w[4 * blk:4 * blk + 4]) == list(oracle.philox4x32_10([blk, 0, 0, 0], key))
    # the counter's high word carries i / 4 beyond 32 bits
    i0 = (1 << 34) + 8
    assert list(oracle.sr_words(seed, 4, start=i0)) == list(oracle.philox4x32_10([2, 1, 0, 0], key))
    assert list(oracle.sr_words(seed, 6, start=5)) == list(w[5:11])


@pytest.mark.parametrize("fmt", FMTS)
def test_cast_matches_exact_brute_force(fmt):
    rng = np.random.default_rng(11)
    n = 3000
    # values spread over the whole grid and beyond: v = u * 2^k, scale exponent e
    u = rng.uniform(-1.0, 1.0, n).astype(np.float32).astype(np.float64)
    k = rng.integers(-12, EMAX[fmt] + 2, n)
    v = np.ldexp(u, k)
    e = rng.integers(-3, 3, n).astype(np.int32)
    r = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    want, Fs = zip(*[brute_sr(float(v[i]), int(e[i]), int(r[i]), fmt) for i in range(n)])
    got = oracle.cast_sr(v, e, r, fmt)
    assert list(got) == list(want)
    # the decision boundary: r = F - 1 rounds up, r = F rounds down (both sides of F)
    idx = [i for i in range(n) if Fs[i] is not None and 1 <= Fs[i] < 2 ** 32 - 1][:500]
    assert len(idx) > 100
    for d in (-1, 0, 1):
        rr = np.array([Fs[i] + d for i in idx], dtype=np.uint64).astype(np.uint32)
        want_d = [brute_sr(float(v[i]), int(e[i]), int(rr[j]), fmt)[0] for j, i in enumerate(idx)]
        assert list(oracle.cast_sr(v[idx], e[idx], rr, fmt)) == want_d


@pytest.mark.parametrize("fmt", FMTS)
def test_grid_values_never_move(fmt):
    g = GRID[fmt]
    vals = np.array([float(x) for x in g] + [-float(x) for x in g[1:]])
    codes = list(range(len(g))) + [c | SIGN[fmt] for c in range(1, len(g))]
    for e in (-5, 0, 7):
        for r in (0, 1, 2 ** 31, 2 ** 32 - 1):
            got = oracle.cast_sr(np.ldexp(vals, e), np.int32(e), np.uint32(r), fmt)
            assert list(got) == codes


@pytest.mark.parametrize("fmt,q", [("e2m1", 0.3), ("e2m1", 1.3), ("e2m1", 2.7), ("e2m1", 4.9), ("e2m1", -5.99),
                                   ("e4m3", 0.0123), ("e4m3", 17.3), ("e4m3", 300.0), ("e5m2", 1e-5), ("e5m2", 9.9)])
def test_unbiased(fmt, q):
    n = 1 << 16
    r = oracle.sr_words(1234, n)
    vals = oracle.decode(oracle.cast_sr(np.full(n, q), np.int32(0), r, fmt), fmt)
    a = abs(q)
    i = bisect.bisect_right(GRID[fmt], Fraction(a)) - 1
    gap = float(GRID[fmt][i + 1] - GRID[fmt][i])
    assert set(np.unique(np.abs(vals))) <= {float(GRID[fmt][i]), float(GRID[fmt][i + 1])}
    se = 0.5 * gap / np.sqrt(n)
    assert abs(vals.mean() - q) < 5 * se


def _bits(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, (rows, cols)) * 1e-3
    x[:, 3] *= 50.0
    import torch
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rotate", [False, True])
def test_quantizer_invariants(fmt, rotate):
    x = _bits(96, 40, 5)
    rows, cols = x.shape
    mask = 0x9E3779B9
    ref_c, ref_s = (oracle.hadamard32_quantize(x, fmt, mask) if rotate else oracle.quantize_transpose(x, fmt))
    c1, s1 = oracle.quantize_transpose_sr(x, fmt, 77, rotate, mask)
    c2, s2 = oracle.quantize_transpose_sr(x, fmt, 77, rotate, mask)
    c3, _ = oracle.quantize_transpose_sr(x, fmt, 78, rotate, mask)
    assert np.array_equal(s1, ref_s), "the scales are the round-to-nearest path's"
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2), "same seed, same result"
    assert not np.array_equal(c1, c3), "another seed rounds differently somewhere"

    # element values before the cast, in output order [cols x rows]
    vals = workloads.bf16_bits_to_f32(x).astype(np.float32)
    if rotate:
        vals = np.stack([np.concatenate([oracle.hadamard32_f32(vals[32 * b:32 * b + 32, c], mask)
                                         for b in range(rows // 32)]) for c in range(cols)])
    else:
        vals = vals.T.copy()
    e = np.repeat(ref_s.astype(np.int32) - 127, 32, axis=1)
    unpack = (lambda c: np.stack([c & 0xF, c >> 4], -1).reshape(c.shape[0], -1)) if fmt == "e2m1" else (lambda c: c)
    got = unpack(c1).ravel()
    down = oracle.cast_sr(vals.ravel(), e.ravel(), np.uint32(2 ** 32 - 1), fmt)
    up = oracle.cast_sr(vals.ravel(), e.ravel(), np.uint32(0), fmt)
    assert np.all((got == down) | (got == up)), "each code is a neighbour of the exact value"
    assert np.any(got != down) and np.any(got != up)
    # the documented word of each element: output index c * rows + t
    r = oracle.sr_words(77, rows * cols)
    assert np.array_equal(got, oracle.cast_sr(vals.ravel(), e.ravel(), r, fmt))


def test_mean_over_seeds_converges():
    """averaging the dequantized result over seeds shrinks the error of every
    element below the saturation point (no bias there); elements in
    (6, 8) * 2^e, which the floor scale rule lets exceed E2M1's largest
    normal, saturate whatever the random word, so their error stays"""
    x = _bits(64, 32, 9)
    exact = workloads.bf16_bits_to_f32(x).astype(np.float64).T
    sc = oracle.quantize_transpose(x, "e2m1")[1]
    sat = np.abs(exact / np.repeat(2.0 ** (sc.astype(np.int64) - 127), 32, axis=1)) > 6
    assert sat.any()
    acc = np.zeros_like(exact)
    for s in range(64):
        c, sc_sr = oracle.quantize_transpose_sr(x, "e2m1", s)
        d = oracle.dequantize(c, sc_sr, "e2m1")
        acc += d
        if s == 0:
            err0 = np.linalg.norm((d - exact)[~sat])
            assert np.array_equal(d[sat], np.sign(exact[sat]) * 6 * 2.0 ** (np.repeat(
                sc.astype(np.int64) - 127, 32, axis=1)[sat]))
    err64 = np.linalg.norm((acc / 64 - exact)[~sat])
    assert err64 < err0 / 4  # ~1/8 expected for 64 independent draws
