"""GPU parity of the K-panel code layout: the transposed quantizers writing
their codes in panels (mx_quantize_transpose_panels,
mx_hadamard32_quantize_panels, the panel modes of mx_quantize_pair), the
fused dual quantizer writing both forms in panels (mx_quantize_dual_panels)
and the GEMM reading them in place (mx_gemm_layout).

A panel operand of R rows and K elements holds K / P panels of R x 128 code
bytes (P = 128 elements for FP8, 256 for E2M1): byte j of row r in panel p is
byte 128 p + j of that row in the row-major layout.  So the oracle's row-major
codes, cut into [R x K/P x 128] and transposed to [K/P x R x 128], are what
the panel quantizers must write, byte for byte; scales stay row-major and must
equal the oracle's.  The GEMM on panel operands must satisfy the same
tolerance as mx_gemm against the oracle and, reading the same bytes in the
same order, give exactly mx_gemm's output.  Covered: every format, with and
without the rotation, ragged column tails, each operand alone in panels and
both, ragged M and N, bf16 and fp32 output, the carrier's byte-0 block check
reading panel codes, the rejections of the layout call, and the full-size
rotated MXFP4 weight-gradient GEMM (14336 x 4096 x 8192), every element.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import check_gemm, to_dev_bf16, to_dev_u8, to_host

pytestmark = pytest.mark.gpu
FMTS = ("e4m3", "e5m2", "e2m1")
MASK = 0x9E3779B9


@pytest.fixture(scope="module")
def mx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_block_amax_amd as m
    m.lib()
    return m


def panel_elems(fmt):
    return 256 if fmt == "e2m1" else 128


def to_panels(codes: np.ndarray) -> np.ndarray:
    """row-major codes [R x Kbytes] -> K-panel layout [Kbytes/128 x R x 128]"""
    r, kb = codes.shape
    assert kb % 128 == 0
    return np.ascontiguousarray(codes.reshape(r, kb // 128, 128).transpose(1, 0, 2))


def _bf16_bits(rng, rows, cols):
    """normal values with ~1% of entries x40, rounded to bf16 (nearest, ties to even)"""
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    v[rng.random((rows, cols)) < 0.01] *= 40.0
    u = v.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _eq(got, want_codes, want_scales, what):
    c, s = to_host(got[0]), to_host(got[1])
    assert s.shape == want_scales.shape and np.array_equal(s, want_scales), "%s: scales differ" % what
    assert c.shape == want_codes.shape and np.array_equal(c, want_codes), "%s: codes differ" % what


# (rows, cols): rows span several panels; ragged column tails against the 64-column tile
QSHAPES = ((512, 300), (1024, 1030), (256, 64))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("shape", QSHAPES)
def test_panel_quantizers_match_oracle(mx, fmt, rotate, shape):
    rows, cols = shape
    rng = np.random.default_rng(rows + cols + 7 * FMTS.index(fmt) + int(rotate))
    x = _bf16_bits(rng, rows, cols)
    d = to_dev_bf16(x)
    print("case", fmt, "rotate" if rotate else "plain", shape, flush=True)
    want = oracle.hadamard32_quantize(x, fmt, MASK) if rotate else oracle.quantize_transpose(x, fmt)
    got = (mx.hadamard32_quantize(d, fmt, MASK, layout="panels") if rotate
           else mx.quantize_transpose(d, fmt, layout="panels"))
    assert tuple(got[0].shape) == (mx.code_cols(rows, fmt) // 128, cols, 128)
    _eq(got, to_panels(want[0]), want[1], "panel quantizer vs oracle")


@pytest.mark.parametrize("pad", [56, 3])
def test_panel_quantizer_strided_input_and_empty(mx, pad):
    """inputs with a row stride above their width: 256 elements (the vectorised
    path) and 203 elements (not a multiple of 4: the general, unvectorised path,
    whose stores go byte by byte), for the rotated quantizer and the dual; and an
    empty input"""
    import torch
    rng = np.random.default_rng(5 + pad)
    x = _bf16_bits(rng, 256, 200)
    full = to_dev_bf16(np.concatenate([x, np.zeros((256, pad), np.uint16)], axis=1))
    view = full[:, :200]
    assert view.stride(0) == 200 + pad
    want = oracle.hadamard32_quantize(x, "e2m1", MASK)
    _eq(mx.hadamard32_quantize(view, "e2m1", MASK, layout="panels"), to_panels(want[0]), want[1], "strided input")
    # the dual: a row form of 200 columns is not whole panels, so its input keeps 256 columns
    xd = _bf16_bits(rng, 256, 256)
    fulld = to_dev_bf16(np.concatenate([xd, np.zeros((256, pad), np.uint16)], axis=1))
    cr, sr, ct, st = mx.quantize_dual(fulld[:, :256], "e4m3", "e2m1", True, MASK, layout="panels")
    wr, wt = oracle.quantize(xd, "e4m3"), oracle.hadamard32_quantize(xd, "e2m1", MASK)
    _eq((cr, sr), to_panels(wr[0]), wr[1], "dual row form, strided input")
    _eq((ct, st), to_panels(wt[0]), wt[1], "dual transposed form, strided input")
    empty = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    c, s = mx.quantize_transpose(empty, "e4m3", layout="panels")
    assert c.numel() == 0 and s.numel() == 0


def test_panel_quantizer_rejects_ragged_panels(mx):
    import torch
    x = torch.zeros((384, 64), dtype=torch.bfloat16, device="cuda")  # 1.5 E2M1 panels
    with pytest.raises(mx.MXError):
        mx.quantize_transpose(x, "e2m1", layout="panels")
    with pytest.raises(ValueError):
        mx.quantize_transpose(x, "e4m3", layout="tiles")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", ["transpose_panels", "hadamard_panels"])
def test_pair_panel_modes(mx, fmt, mode):
    """both tensors in one launch, different shapes (the second grid row range
    outruns the shorter tensor), each equal to the oracle in panels and to the
    single panel call"""
    rng = np.random.default_rng(11 + FMTS.index(fmt) + (3 if mode.startswith("h") else 0))
    x0, x1 = _bf16_bits(rng, 1024, 300), _bf16_bits(rng, 256, 260)
    d0, d1 = to_dev_bf16(x0), to_dev_bf16(x1)
    rot = mode.startswith("hadamard")
    print("case", mode, fmt, flush=True)
    p0, p1 = mx.quantize_pair(mode, d0, d1, fmt, MASK)
    for p, x, d, what in ((p0, x0, d0, "first"), (p1, x1, d1, "second")):
        want = oracle.hadamard32_quantize(x, fmt, MASK) if rot else oracle.quantize_transpose(x, fmt)
        _eq(p, to_panels(want[0]), want[1], "%s tensor vs oracle" % what)
        single = (mx.hadamard32_quantize(d, fmt, MASK, layout="panels") if rot
                  else mx.quantize_transpose(d, fmt, layout="panels"))
        _eq(p, to_host(single[0]), to_host(single[1]), "%s tensor vs single call" % what)


DUAL_FMTS = [("e2m1", "e2m1"), ("e4m3", "e4m3"), ("e4m3", "e2m1"), ("e2m1", "e5m2")]


@pytest.mark.parametrize("fr,ft", DUAL_FMTS)
@pytest.mark.parametrize("rotate", [False, True])
def test_dual_panels_match_oracle(mx, fr, ft, rotate):
    """mx_quantize_dual_panels: the row form and the (rotated) transposed form, each
    equal to the oracle's codes cut into panels and to its scales, for row counts of
    several workgroup row spans; with an FP8 row form, 640 columns leave the last
    256-column tile half full"""
    rng = np.random.default_rng(31 + DUAL_FMTS.index((fr, ft)) * 2 + int(rotate))
    rows, cols = 512, (768 if fr == "e2m1" else 640)
    x = _bf16_bits(rng, rows, cols)
    print("case", fr, ft, "rotate" if rotate else "plain", flush=True)
    cr, sr, ct, st = mx.quantize_dual(to_dev_bf16(x), fr, ft, rotate, MASK, layout="panels")
    wr = oracle.quantize(x, fr)
    wt = oracle.hadamard32_quantize(x, ft, MASK) if rotate else oracle.quantize_transpose(x, ft)
    _eq((cr, sr), to_panels(wr[0]), wr[1], "row form")
    _eq((ct, st), to_panels(wt[0]), wt[1], "transposed form")


def _rand_operand(rng, rows, K, fmt):
    v = rng.standard_t(4, (rows, K)) * np.exp2(rng.integers(-6, 6, (rows, K // 32))).repeat(32, 1)
    u = v.astype(np.float32).view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return oracle.quantize(bits, fmt)


def _host_c(c, bf16):
    h = to_host(c)
    return workloads.bf16_bits_to_f32(h).astype(np.float64) if bf16 else h.astype(np.float64)


# (fa, fb, which operands in panels): both E2M1 (the scaled FP4 kernel), FP8 pairs on
# the carrier with either or both operands in panels, and an FP8 panel operand beside
# a row-major E2M1 one, as A and as B
GCASES = [("e2m1", "e2m1", (1, 1)), ("e2m1", "e2m1", (1, 0)), ("e2m1", "e2m1", (0, 1)),
          ("e4m3", "e4m3", (1, 1)), ("e5m2", "e4m3", (0, 1)), ("e4m3", "e2m1", (1, 0)),
          ("e2m1", "e5m2", (0, 1))]


@pytest.mark.parametrize("fa,fb,pan", GCASES)
@pytest.mark.parametrize("bf16", [False, True])
def test_gemm_layout_matches_oracle_and_row_major(mx, fa, fb, pan, bf16):
    import torch
    M, N, K = 300, 520, 1024
    rng = np.random.default_rng(GCASES.index((fa, fb, pan)) * 2 + int(bf16))
    qa, qb = _rand_operand(rng, M, K, fa), _rand_operand(rng, N, K, fb)
    C, S = oracle.gemm(qa[0], qa[1], fa, qb[0], qb[1], fb)
    dt = torch.bfloat16 if bf16 else torch.float32
    ac = to_dev_u8(to_panels(qa[0]) if pan[0] else qa[0])
    bc = to_dev_u8(to_panels(qb[0]) if pan[1] else qb[0])
    print("case", fa, fb, pan, "bf16" if bf16 else "f32", flush=True)
    c = mx.gemm(ac, to_dev_u8(qa[1]), fa, bc, to_dev_u8(qb[1]), fb, out_dtype=dt)
    r = check_gemm(_host_c(c, bf16), C, S, bf16)
    dense = mx.gemm(to_dev_u8(qa[0]), to_dev_u8(qa[1]), fa, to_dev_u8(qb[0]), to_dev_u8(qb[1]), fb, out_dtype=dt)
    assert torch.equal(c.view(torch.int16 if bf16 else torch.int32), dense.view(torch.int16 if bf16 else torch.int32))
    print("max |err|/S", r, flush=True)


def _random_codes(rng, rows, K, fmt):
    """uniform random code bytes; FP8 NaN (E4M3) and Inf/NaN (E5M2) codes replaced by 1.0"""
    if fmt == "e2m1":
        return rng.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    c = rng.integers(0, 256, (rows, K)).astype(np.uint8)
    c[((c & 0x7F) == 0x7F) if fmt == "e4m3" else ((c & 0x7C) == 0x7C)] = 0x38
    return c


@pytest.mark.parametrize("fa,fb,pan", [("e4m3", "e4m3", (1, 1)), ("e5m2", "e4m3", (0, 1)), ("e4m3", "e2m1", (1, 0))])
@pytest.mark.parametrize("case", ["zero_blocks", "tiny_blocks"])
def test_gemm_layout_carrier_blocks_under_scale_zero(mx, fa, fb, pan, case):
    """the carrier's pre-check reads the codes of byte-0 blocks (rows whose other
    blocks lie 100+ binades higher) in the panel layout: all-zero blocks keep the
    fast path, blocks of tiny nonzero values must send their tile to the exact
    kernel; C within the tolerance of the oracle and equal to mx_gemm's on the
    row-major codes"""
    import torch
    rng = np.random.default_rng(71 + ["zero_blocks", "tiny_blocks"].index(case) * 10 + FMTS.index(fa) + 3 * FMTS.index(fb))
    M, N, K = 300, 272, 1024
    kb = K // 32
    ca, cb = _random_codes(rng, M, K, fa), _random_codes(rng, N, K, fb)
    sa = rng.integers(98, 128, (M, kb)).astype(np.uint8)
    sb = rng.integers(98, 128, (N, kb)).astype(np.uint8)
    for c, s, fmt, rows in ((ca, sa, fa, np.arange(0, M, 2)), (cb, sb, fb, np.arange(1, N, 5))):
        nb = 16 if fmt == "e2m1" else 32
        for r, b in zip(rows, rng.integers(0, kb, rows.size)):
            s[r, b] = 0
            c[r, b * nb:(b + 1) * nb] = (0x88 if fmt == "e2m1" else 0x80) if r % 3 == 0 else 0
    if case == "tiny_blocks":
        for r in (4, 130, 262):
            sa[r, int(rng.integers(0, kb))] = 0
    C, S = oracle.gemm(ca, sa, fa, cb, sb, fb)
    print("case", case, fa, fb, pan, flush=True)
    for bf16 in (False, True):
        dt = torch.bfloat16 if bf16 else torch.float32
        got = mx.gemm(to_dev_u8(to_panels(ca) if pan[0] else ca), to_dev_u8(sa), fa,
                      to_dev_u8(to_panels(cb) if pan[1] else cb), to_dev_u8(sb), fb, out_dtype=dt)
        dense = mx.gemm(to_dev_u8(ca), to_dev_u8(sa), fa, to_dev_u8(cb), to_dev_u8(sb), fb, out_dtype=dt)
        iv = torch.int16 if bf16 else torch.int32
        assert torch.equal(got.view(iv), dense.view(iv))
        r = check_gemm(_host_c(got, bf16), C, S, bf16)
        print(case, "bf16" if bf16 else "f32", "max |err|/S", r, flush=True)


def test_gemm_layout_k_zero(mx):
    """K = 0 with panel operands (no panels at all): C = 0, as mx_gemm writes it"""
    import torch
    M, N = 70, 300
    a = torch.empty((0, M, 128), dtype=torch.uint8, device="cuda")
    b = torch.empty((0, N, 128), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, 0), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N, 0), dtype=torch.uint8, device="cuda")
    out = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    c = mx.gemm(a, sa, "e2m1", b, sb, "e2m1", out_dtype=torch.float32, out=out)
    assert torch.count_nonzero(c).item() == 0


def test_gemm_layout_rows_is_mx_gemm_and_rejections(mx):
    """both operands row-major through mx_gemm_layout is mx_gemm (any K); panel
    operands on shapes the pipelined kernel does not take are rejected"""
    import ctypes
    import torch
    rng = np.random.default_rng(3)
    M, N, K = 70, 90, 352
    qa, qb = _rand_operand(rng, M, K, "e4m3"), _rand_operand(rng, N, K, "e5m2")
    dev = [to_dev_u8(t) for t in (qa[0], qa[1], qb[0], qb[1])]
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    L = mx.lib()
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.mx_gemm_layout(ptr(dev[0]), 0, ptr(dev[1]), mx.E4M3, ptr(dev[2]), 0, ptr(dev[3]), mx.E5M2, M, N, K,
                          ptr(out), mx.OUT_F32, N, None)
    assert st == 0
    want = mx.gemm(*dev[:2], "e4m3", *dev[2:], "e5m2", out_dtype=torch.float32)
    assert torch.equal(out.view(torch.int32), want.view(torch.int32))
    # K = 352 is not a multiple of 512: a panel operand is unsupported
    st = L.mx_gemm_layout(ptr(dev[0]), 1, ptr(dev[1]), mx.E4M3, ptr(dev[2]), 0, ptr(dev[3]), mx.E5M2, M, N, K,
                          ptr(out), mx.OUT_F32, N, None)
    assert st == 2
    # an E2M1 panel operand beside an FP8 one is unsupported
    qa4 = _rand_operand(rng, M, 512, "e2m1")
    qb8 = _rand_operand(rng, N, 512, "e4m3")
    a4, as4, b8, bs8 = (to_dev_u8(t) for t in (to_panels(qa4[0]), qa4[1], qb8[0], qb8[1]))
    with pytest.raises(mx.MXError):
        mx.gemm(a4, as4, "e2m1", b8, bs8, "e4m3")


def test_full_size_rotated_wgrad_in_panels(mx):
    """the rotated MXFP4 weight-gradient GEMM of the Llama-3.1-8B down projection at
    full size (M 14336, N 4096, K 8192 tokens): both operands quantized by the GPU in
    one launch straight into panels, equal to the oracle's codes on every byte; the
    GEMM on them equal to mx_gemm on the row-major codes and, every element, within
    the tolerance of the oracle's product"""
    import torch
    cfg = workloads.config(3)
    g = cfg.gemms[0]
    qa_spec, qb_spec = cfg.quant(g.a), cfg.quant(g.b)
    xa = workloads.draw_tensor(cfg, qa_spec.tensor)
    xb = workloads.draw_tensor(cfg, qb_spec.tensor)
    print("case", cfg.name, g.name, g.M, g.N, g.K, flush=True)
    (ac, as_), (bc, bs) = mx.quantize_pair("hadamard_panels", to_dev_bf16(xa), to_dev_bf16(xb), "e2m1",
                                          qa_spec.sign_mask)
    qa = oracle.hadamard32_quantize(xa, "e2m1", qa_spec.sign_mask)
    qb = oracle.hadamard32_quantize(xb, "e2m1", qb_spec.sign_mask)
    _eq((ac, as_), to_panels(qa[0]), qa[1], "dY operand")
    _eq((bc, bs), to_panels(qb[0]), qb[1], "X operand")
    print("operands equal to the oracle", flush=True)
    c = mx.gemm(ac, as_, "e2m1", bc, bs, "e2m1", out_dtype=torch.float32)
    dense = mx.gemm(to_dev_u8(qa[0]), as_, "e2m1", to_dev_u8(qb[0]), bs, "e2m1", out_dtype=torch.float32)
    assert torch.equal(c.view(torch.int32), dense.view(torch.int32))
    ch = _host_c(c, False)
    worst = 0.0
    for r0 in range(0, g.M, 2048):
        rows = np.arange(r0, min(g.M, r0 + 2048))
        C, S = oracle.gemm(qa[0], qa[1], "e2m1", qb[0], qb[1], "e2m1", rows=rows)
        worst = max(worst, check_gemm(ch[rows], C, S, False))
        print("rows %d..%d checked" % (rows[0], rows[-1]), flush=True)
    print("max |err|/S", worst, flush=True)
