"""GPU parity of the three quantizers against the oracle: codes and scales bit-exact.

Inputs are the seeded workloads at their full sizes plus edge suites (zero,
subnormal, tie, saturation, non-finite blocks), ragged / strided / unaligned
layouts, empty inputs, guard bands around outputs, and repeat-run determinism.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import to_dev_bf16, to_dev_u8, to_host

pytestmark = pytest.mark.gpu
FMTS = ("e4m3", "e5m2", "e2m1")


@pytest.fixture(scope="module")
def mx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_block_amax_amd as m
    m.lib()
    return m


def _cmp(got, want, what):
    g, w = to_host(got[0]), to_host(got[1])
    bad_c = np.nonzero(g != want[0])
    bad_s = np.nonzero(w != want[1])
    assert bad_s[0].size == 0, "%s: scale mismatch at %s gpu %d oracle %d (%d bad)" % (
        what, tuple(b[0] for b in bad_s), w[tuple(b[0] for b in bad_s)], want[1][tuple(b[0] for b in bad_s)], bad_s[0].size)
    assert bad_c[0].size == 0, "%s: code mismatch at %s gpu %#x oracle %#x (%d bad)" % (
        what, tuple(b[0] for b in bad_c), g[tuple(b[0] for b in bad_c)], want[0][tuple(b[0] for b in bad_c)], bad_c[0].size)


ROW_CASES = [(0, "A", "e4m3"), (0, "A", "e5m2"), (0, "A", "e2m1"),
             (1, "X", "e4m3"), (1, "W", "e4m3"), (2, "X", "e2m1"), (2, "W", "e2m1")]


@pytest.mark.parametrize("ci,name,fmt", ROW_CASES)
def test_row_quantize_workloads(mx, ci, name, fmt):
    cfg = workloads.config(ci)
    x = workloads.draw_tensor(cfg, name)
    print("case", cfg.name, name, fmt, x.shape, flush=True)
    got = mx.quantize(to_dev_bf16(x), fmt)
    _cmp(got, oracle.quantize(x, fmt), "%s/%s" % (cfg.name, name))


TR_CASES = [(0, "B", "e4m3"), (0, "B", "e5m2"), (0, "B", "e2m1"), (3, "X", "e2m1")]


@pytest.mark.parametrize("ci,name,fmt", TR_CASES)
def test_transpose_quantize_workloads(mx, ci, name, fmt):
    cfg = workloads.config(ci)
    x = workloads.draw_tensor(cfg, name)
    print("case", cfg.name, name, fmt, x.shape, flush=True)
    got = mx.quantize_transpose(to_dev_bf16(x), fmt)
    _cmp(got, oracle.quantize_transpose(x, fmt), "%s/%s" % (cfg.name, name))


H_CASES = [(3, "dY", "e2m1", 0), (3, "X", "e2m1", 0), (3, "dY", "e2m1", 0x9E3779B9),
           (3, "X", "e4m3", 0x9E3779B9), (0, "B", "e5m2", 0xFFFFFFFF)]


@pytest.mark.parametrize("ci,name,fmt,mask", H_CASES)
def test_hadamard_quantize_workloads(mx, ci, name, fmt, mask):
    cfg = workloads.config(ci)
    x = workloads.draw_tensor(cfg, name)
    print("case", cfg.name, name, fmt, hex(mask), x.shape, flush=True)
    got = mx.hadamard32_quantize(to_dev_bf16(x), fmt, mask)
    _cmp(got, oracle.hadamard32_quantize(x, fmt, mask), "%s/%s" % (cfg.name, name))


def edge_matrix(rows=64, cols=256, seed=5):
    """bf16 bits mixing every edge: zero / -0 / subnormal / huge / tie-rich /
    non-finite blocks, at random positions, over a normal background"""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((rows, cols)).astype(np.float32)
    import torch
    bits = torch.from_numpy(base).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    kinds = [
        lambda n: np.zeros(n, dtype=np.uint16),
        lambda n: np.full(n, 0x8000, dtype=np.uint16),
        lambda n: rng.integers(0, 0x80, n).astype(np.uint16),
        lambda n: (rng.integers(0, 0x80, n) | 0x8000).astype(np.uint16),
        lambda n: rng.integers(0x7F00, 0x7F80, n).astype(np.uint16),
        lambda n: rng.integers(0x3F00, 0x4100, n).astype(np.uint16),
        lambda n: rng.integers(0, 0x7F80, n).astype(np.uint16) | (rng.integers(0, 2, n) << 15).astype(np.uint16),
        lambda n: np.where(rng.random(n) < 0.1, 0x7F80, 0x3F80).astype(np.uint16),
        lambda n: np.where(rng.random(n) < 0.1, 0xFFC1, 0x4000).astype(np.uint16),
    ]
    return bits, kinds, rng


def edge_rows(rows=64, cols=256):
    bits, kinds, rng = edge_matrix(rows, cols)
    for r in range(rows):
        for b in range(cols // 32):
            k = rng.integers(0, len(kinds) + 3)
            if k < len(kinds):
                bits[r, 32 * b:32 * b + 32] = kinds[k](32)
    return bits


def edge_cols(rows=256, cols=64):
    bits, kinds, rng = edge_matrix(rows, cols, seed=6)
    for c in range(cols):
        for b in range(rows // 32):
            k = rng.integers(0, len(kinds) + 3)
            if k < len(kinds):
                bits[32 * b:32 * b + 32, c] = kinds[k](32)
    return bits


@pytest.mark.parametrize("fmt", FMTS)
def test_edge_suite_row(mx, fmt):
    x = edge_rows()
    _cmp(mx.quantize(to_dev_bf16(x), fmt), oracle.quantize(x, fmt), "edge rows")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rotate", [False, True])
def test_edge_suite_transposed(mx, fmt, rotate):
    x = edge_cols()
    if rotate:
        for mask in (0, 0x9E3779B9):
            _cmp(mx.hadamard32_quantize(to_dev_bf16(x), fmt, mask), oracle.hadamard32_quantize(x, fmt, mask),
                 "edge rotate")
    else:
        _cmp(mx.quantize_transpose(to_dev_bf16(x), fmt), oracle.quantize_transpose(x, fmt), "edge transposed")


def _rand_bits(rows, cols, seed):
    import torch
    rng = np.random.default_rng(seed)
    v = (rng.standard_t(4, (rows, cols)) * np.exp2(rng.integers(-8, 8, (rows, 1)))).astype(np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,cols,extra", [(1, 32, 0), (3, 96, 0), (97, 224, 0), (5, 4128, 0),
                                             (33, 64, 8), (7, 160, 3), (130, 1056, 40)])
def test_row_ragged_strided(mx, fmt, rows, cols, extra):
    full = _rand_bits(rows, cols + extra, rows * 1000 + cols)
    xd = to_dev_bf16(full)[:, :cols]        # strided view when extra > 0 (extra odd: unaligned rows)
    _cmp(mx.quantize(xd, fmt), oracle.quantize(np.ascontiguousarray(full[:, :cols]), fmt), "ragged rows")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("rows,cols,extra", [(32, 1, 0), (64, 37, 0), (96, 255, 0), (160, 258, 0),
                                             (32, 1030, 0), (64, 16, 5), (224, 300, 2),
                                             (544, 300, 0), (800, 1030, 2), (1056, 260, 4)])
def test_transposed_ragged_strided(mx, fmt, rotate, rows, cols, extra):
    """ragged and strided shapes; the last three span several workgroup row groups
    (8 or 16 row blocks each) with a partial last group"""
    full = _rand_bits(rows, cols + extra, rows * 7 + cols)
    xd = to_dev_bf16(full)[:, :cols]
    x = np.ascontiguousarray(full[:, :cols])
    if rotate:
        _cmp(mx.hadamard32_quantize(xd, fmt, 0x12345678), oracle.hadamard32_quantize(x, fmt, 0x12345678), "ragged H")
    else:
        _cmp(mx.quantize_transpose(xd, fmt), oracle.quantize_transpose(x, fmt), "ragged T")


@pytest.mark.parametrize("fmt", FMTS)
def test_unaligned_pointers(mx, fmt):
    import torch
    x = _rand_bits(64, 128, 99)
    buf = torch.empty(64 * 128 + 1, dtype=torch.bfloat16, device="cuda")
    xd = buf[1:].view(64, 128)                 # 2-byte aligned input
    xd.copy_(to_dev_bf16(x))
    nb = 64 * 128 // (2 if fmt == "e2m1" else 1)
    cbuf = torch.empty(nb + 3, dtype=torch.uint8, device="cuda")
    codes = cbuf[3:].view(64, nb // 64)        # odd code pointer
    scales = torch.empty(64, 4, dtype=torch.uint8, device="cuda")
    mx.quantize(xd, fmt, out=(codes, scales))
    _cmp((codes, scales), oracle.quantize(x, fmt), "unaligned rows")
    nbt = 128 * 64 // (2 if fmt == "e2m1" else 1)
    cbuf2 = torch.empty(nbt + 1, dtype=torch.uint8, device="cuda")
    codes_t = cbuf2[1:].view(128, nbt // 128)
    scales_t = torch.empty(128, 2, dtype=torch.uint8, device="cuda")
    mx.quantize_transpose(xd, fmt, out=(codes_t, scales_t))
    _cmp((codes_t, scales_t), oracle.quantize_transpose(x, fmt), "unaligned transposed")


def test_empty_inputs(mx):
    import torch
    for fn in (mx.quantize, mx.quantize_transpose, mx.hadamard32_quantize):
        c, s = fn(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"), "e4m3")
        assert c.numel() == 0 or c.shape[1] == 0
    c, s = mx.quantize(torch.empty(4, 0, dtype=torch.bfloat16, device="cuda"), "e2m1")
    assert c.shape == (4, 0) and s.shape == (4, 0)


@pytest.mark.parametrize("kind", ["row", "transpose", "hadamard"])
def test_guard_bands(mx, kind):
    """outputs written exactly in place: sentinels before and after stay intact"""
    import torch
    x = _rand_bits(128, 256, 3)
    xd = to_dev_bf16(x)
    fmt = "e2m1"
    rows_out, k = (128, 256) if kind == "row" else (256, 128)
    nc, ns, g = rows_out * k // 2, rows_out * k // 32, 4096
    cb = torch.full((nc + 2 * g,), 0xA5, dtype=torch.uint8, device="cuda")
    sb = torch.full((ns + 2 * g,), 0x5A, dtype=torch.uint8, device="cuda")
    out = (cb[g:g + nc].view(rows_out, k // 2), sb[g:g + ns].view(rows_out, k // 32))
    if kind == "row":
        mx.quantize(xd, fmt, out=out)
        want = oracle.quantize(x, fmt)
    elif kind == "transpose":
        mx.quantize_transpose(xd, fmt, out=out)
        want = oracle.quantize_transpose(x, fmt)
    else:
        mx.hadamard32_quantize(xd, fmt, 0, out=out)
        want = oracle.hadamard32_quantize(x, fmt, 0)
    _cmp(out, want, "guard " + kind)
    c, s = to_host(cb), to_host(sb)
    assert np.all(c[:g] == 0xA5) and np.all(c[g + nc:] == 0xA5)
    assert np.all(s[:g] == 0x5A) and np.all(s[g + ns:] == 0x5A)


def test_repeat_and_streams_deterministic(mx):
    import torch
    cfg = workloads.config(3)
    x = to_dev_bf16(workloads.draw_tensor(cfg, "dY", rows=(0, 1024)))
    ref = [to_host(t) for t in mx.hadamard32_quantize(x, "e2m1", 0x9E3779B9)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            got = [to_host(t) for t in mx.hadamard32_quantize(x, "e2m1", 0x9E3779B9)]
            assert all(np.array_equal(a, b) for a, b in zip(ref, got))
    torch.cuda.synchronize()


def test_bad_arguments_raise(mx):
    import torch
    x = torch.zeros(64, 48, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mx.MXError):
        mx.quantize(x, "e4m3")                  # cols % 32 != 0
    with pytest.raises(mx.MXError):
        mx.quantize_transpose(x[:40], "e4m3")   # rows % 32 != 0


EMAX = {"e4m3": 8, "e5m2": 15, "e2m1": 2}


def exhaustive_blocks(fmt):
    """Every finite bf16 value at every reachable block scale exponent e.

    For each e, blocks lead with the largest bf16 of the binade [2^(e+emax),
    2^(e+emax+1)) (alternating sign), which fixes the block's scale at e; the
    other 31 elements run through every finite bf16 pattern of either sign
    whose magnitude does not exceed it (zeros pad the last block).  Returns a
    [rows x 4096] bf16 bit matrix of whole blocks."""
    em = EMAX[fmt]
    mags = np.arange(0x7F80, dtype=np.uint32)
    parts = []
    for e in range(-127, 128):
        k = e + em                                   # floor(log2 amax)
        if k > 127 or k < -133:
            continue
        top = ((k + 127) << 7) | 0x7F if k >= -126 else (1 << (k + 134)) - 1
        p = mags[mags <= top]
        vals = np.concatenate([p, p | 0x8000]).astype(np.uint16)
        n = -(-vals.size // 31)
        body = np.zeros(n * 31, np.uint16)
        body[:vals.size] = vals
        head = np.full((n, 1), top, np.uint16)
        head[1::2] |= 0x8000
        parts.append(np.concatenate([head, body.reshape(n, 31)], axis=1))
    b = np.concatenate(parts)
    nb = -(-b.shape[0] // 128) * 128
    out = np.zeros((nb, 32), np.uint16)
    out[:b.shape[0]] = b
    return out.reshape(nb // 128, 4096)


@pytest.mark.parametrize("fmt", FMTS)
def test_every_bf16_at_every_scale(mx, fmt):
    """The element casts (the gfx950 scaled conversion instructions, bf16 form
    in row mode and fp32 form in transposed mode) equal the oracle on every
    finite bf16 input at every reachable scale exponent."""
    x = exhaustive_blocks(fmt)
    want = oracle.quantize(x, fmt)
    _cmp(mx.quantize(to_dev_bf16(x), fmt), want, "row, every bf16 x every e")
    xt = np.ascontiguousarray(x.T)                   # the same blocks, now along rows
    _cmp(mx.quantize_transpose(to_dev_bf16(xt), fmt), oracle.quantize_transpose(xt, fmt),
         "transposed, every bf16 x every e")
    assert np.array_equal(oracle.quantize_transpose(xt, fmt)[0], want[0])


# ---------------------------------------------------------------------------
# Fused dual-direction quantizer: both outputs equal the single-direction oracle forms.

def _cmp_dual(got, x, fr, ft, rotate, mask, what):
    _cmp(got[:2], oracle.quantize(x, fr), what + " (row form)")
    want_t = oracle.hadamard32_quantize(x, ft, mask) if rotate else oracle.quantize_transpose(x, ft)
    _cmp(got[2:], want_t, what + " (transposed form)")


DUAL_CASES = [(1, "X", "e4m3", "e4m3", False, 0), (2, "W", "e2m1", "e2m1", False, 0),
              (3, "dY", "e2m1", "e2m1", True, 0), (3, "X", "e2m1", "e2m1", True, 0x9E3779B9),
              (0, "A", "e5m2", "e4m3", True, 0xFFFFFFFF)]


@pytest.mark.parametrize("ci,name,fr,ft,rotate,mask", DUAL_CASES)
def test_dual_workloads(mx, ci, name, fr, ft, rotate, mask):
    cfg = workloads.config(ci)
    x = workloads.draw_tensor(cfg, name)
    print("case dual", cfg.name, name, fr, ft, rotate, hex(mask), x.shape, flush=True)
    got = mx.quantize_dual(to_dev_bf16(x), fr, ft, rotate, mask)
    _cmp_dual(got, x, fr, ft, rotate, mask, "%s/%s" % (cfg.name, name))


@pytest.mark.parametrize("fr", FMTS)
@pytest.mark.parametrize("ft", FMTS)
@pytest.mark.parametrize("rotate", [False, True])
def test_dual_format_pairs_ragged(mx, fr, ft, rotate):
    """rows and columns not multiples of the workgroup tile (256 x 256)"""
    rng = np.random.default_rng(FMTS.index(fr) * 3 + FMTS.index(ft))
    x = _rand_bits(96 + 32 * FMTS.index(fr), 352 - 32 * FMTS.index(ft), int(rng.integers(1 << 30)))
    mask = 0x9E3779B9 if rotate else 0
    _cmp_dual(mx.quantize_dual(to_dev_bf16(x), fr, ft, rotate, mask), x, fr, ft, rotate, mask, "ragged")


@pytest.mark.parametrize("fmt", FMTS)
def test_dual_edges_strided_unaligned(mx, fmt):
    import torch
    rows_e = edge_rows(64, 256)     # special values along rows
    cols_e = edge_cols(256, 64)     # ... and along columns
    x = np.concatenate([np.concatenate([rows_e, np.zeros((64, 0), np.uint16)], axis=1)[:, :64], cols_e[:64]], axis=0)
    x = np.ascontiguousarray(np.concatenate([x, edge_rows(128, 64)], axis=1)[:, :96])
    _cmp_dual(mx.quantize_dual(to_dev_bf16(x), fmt, fmt, True, 0x12345678), x, fmt, fmt, True, 0x12345678, "edges")
    # strided input (ldx > cols) and misaligned outputs (byte-store path)
    big = _rand_bits(128, 200, 11)
    xs = to_dev_bf16(big)[:, 8:168]
    rows, cols = xs.shape
    raw = torch.empty(4 * rows * cols + 64, dtype=torch.uint8, device="cuda")
    cb = mx.code_cols(cols, fmt) * rows
    ctb = mx.code_cols(rows, fmt) * cols
    off = 1
    cr = raw[off:off + cb].view(rows, -1)
    sr = raw[off + cb:off + cb + rows * cols // 32].view(rows, -1)
    o2 = off + cb + rows * cols // 32 + 3
    ct = raw[o2:o2 + ctb].view(cols, -1)
    st = raw[o2 + ctb:o2 + ctb + rows * cols // 32].view(cols, -1)
    got = mx.quantize_dual(xs, fmt, fmt, False, 0, out=(cr, sr, ct, st))
    _cmp_dual(got, np.ascontiguousarray(big[:, 8:168]), fmt, fmt, False, 0, "strided/unaligned")


@pytest.mark.parametrize("fmt", FMTS)
def test_dual_every_bf16_at_every_scale(mx, fmt):
    x = exhaustive_blocks(fmt)
    x = np.concatenate([x, np.zeros((-x.shape[0] % 32, x.shape[1]), np.uint16)])   # rows to a multiple of 32
    got = mx.quantize_dual(to_dev_bf16(x), fmt, fmt, False, 0)
    _cmp_dual(got, x, fmt, fmt, False, 0, "dual, every bf16 x every e")
