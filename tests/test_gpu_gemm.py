"""GPU parity of mx_gemm against the oracle, within the fp32 accumulation tolerance.

|C_gpu - C_ref| <= 1e-5 * sum_k |a_mk b_nk| per element (plus half a bf16 ulp
when the output is bf16); elements with S_abs = 0 must be exactly 0.  The
operands come from the oracle's own quantization of the seeded inputs, so the
GEMM is checked in isolation; the end-to-end chain (GPU quantizers feeding the
GPU GEMM) is checked too, bit-exact codes being established by the quantizer
tests.  Full-size configurations are compared on every element.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import check_gemm, to_dev_bf16, to_dev_u8, to_host

pytestmark = pytest.mark.gpu
FMTS = ("e4m3", "e5m2", "e2m1")


@pytest.fixture(scope="module")
def mx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_block_amax_amd as m
    m.lib()
    return m


def _run(mx, qa, fa, qb, fb, bf16, out=None):
    import torch
    return mx.gemm(to_dev_u8(qa[0]), to_dev_u8(qa[1]), fa, to_dev_u8(qb[0]), to_dev_u8(qb[1]), fb,
                   out_dtype=torch.bfloat16 if bf16 else torch.float32, out=out)


def _host_c(c, bf16):
    h = to_host(c)
    return workloads.bf16_bits_to_f32(h).astype(np.float64) if bf16 else h.astype(np.float64)


def _oracle_operands(cfg, qname):
    q = cfg.quant(qname)
    x = workloads.draw_tensor(cfg, q.tensor)
    if q.kind == "row":
        return oracle.quantize(x, q.fmt)
    if q.kind == "transpose":
        return oracle.quantize_transpose(x, q.fmt)
    return oracle.hadamard32_quantize(x, q.fmt, q.sign_mask)


def test_small_config_all_elements(mx):
    cfg = workloads.config(0)
    g = cfg.gemms[0]
    qa, qb = _oracle_operands(cfg, g.a), _oracle_operands(cfg, g.b)
    C, S = oracle.gemm(qa[0], qa[1], "e4m3", qb[0], qb[1], "e4m3")
    c = _run(mx, qa, "e4m3", qb, "e4m3", False)
    r = check_gemm(_host_c(c, False), C, S, False)
    print("max |err|/S", r)


def test_small_config_end_to_end(mx):
    """GPU quantizers feeding the GPU GEMM: codes equal the oracle's, C within tolerance"""
    import torch
    cfg = workloads.config(0)
    a = workloads.draw_tensor(cfg, "A")
    b = workloads.draw_tensor(cfg, "B")
    ca, sa = mx.quantize(to_dev_bf16(a), "e4m3")
    cb, sb = mx.quantize_transpose(to_dev_bf16(b), "e4m3")
    c = mx.gemm(ca, sa, "e4m3", cb, sb, "e4m3", out_dtype=torch.float32)
    qa, qb = oracle.quantize(a, "e4m3"), oracle.quantize_transpose(b, "e4m3")
    assert np.array_equal(to_host(ca), qa[0]) and np.array_equal(to_host(sb), qb[1])
    C, S = oracle.gemm(qa[0], qa[1], "e4m3", qb[0], qb[1], "e4m3")
    check_gemm(_host_c(c, False), C, S, False)


@pytest.mark.parametrize("fa,fb,a,b,want", [("e4m3", "e4m3", 1.0, 1.0, 32.0), ("e2m1", "e2m1", 6.0, -0.5, -96.0)])
def test_worked_examples(mx, fa, fb, a, b, want):
    import torch
    xa = torch.full((1, 32), a, dtype=torch.bfloat16, device="cuda")
    xb = torch.full((1, 32), b, dtype=torch.bfloat16, device="cuda")
    ca, sa = mx.quantize(xa, fa)
    cb, sb = mx.quantize(xb, fb)
    c = mx.gemm(ca, sa, fa, cb, sb, fb, out_dtype=torch.float32)
    assert to_host(c)[0, 0] == want


def _rand_operand(rng, rows, K, fmt):
    import torch
    v = (rng.standard_t(4, (rows, K)) * np.exp2(rng.integers(-6, 6, (rows, K // 32))).repeat(32, 1)).astype(np.float32)
    bits = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return oracle.quantize(bits, fmt)


@pytest.mark.parametrize("fa", FMTS)
@pytest.mark.parametrize("fb", FMTS)
@pytest.mark.parametrize("bf16", [False, True])
def test_format_pairs_with_tails(mx, fa, fb, bf16):
    """every format pair; M, N not multiples of the tile; K not a multiple of the K tile"""
    rng = np.random.default_rng(FMTS.index(fa) * 3 + FMTS.index(fb))
    M, N, K = 300, 200, 352
    qa, qb = _rand_operand(rng, M, K, fa), _rand_operand(rng, N, K, fb)
    C, S = oracle.gemm(qa[0], qa[1], fa, qb[0], qb[1], fb)
    check_gemm(_host_c(_run(mx, qa, fa, qb, fb, bf16), bf16), C, S, bf16)


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (33, 17, 64), (256, 512, 32), (512, 256, 1024), (64, 1000, 160)])
def test_shapes(mx, M, N, K):
    rng = np.random.default_rng(M + N + K)
    qa, qb = _rand_operand(rng, M, K, "e4m3"), _rand_operand(rng, N, K, "e2m1")
    C, S = oracle.gemm(qa[0], qa[1], "e4m3", qb[0], qb[1], "e2m1")
    check_gemm(_host_c(_run(mx, qa, "e4m3", qb, "e2m1", False), False), C, S, False)


@pytest.mark.parametrize("fa,fb,K", [("e2m1", "e2m1", 1024), ("e2m1", "e2m1", 1536), ("e4m3", "e4m3", 1536),
                                     ("e4m3", "e2m1", 1024)])
def test_second_round_k_order(mx, fa, fb, K):
    """17 x 17 tiles of 256 x 256: more than one round on 256 CUs, and the
    second round takes K's 16-byte scale slots (512 elements each) in
    descending order: two or three slots of 256-K (E2M1 x E2M1) or 128-K
    stages; every element within the tolerance"""
    rng = np.random.default_rng(K + FMTS.index(fa) * 3 + FMTS.index(fb))
    M = N = 17 * 256
    qa, qb = _rand_operand(rng, M, K, fa), _rand_operand(rng, N, K, fb)
    C, S = oracle.gemm(qa[0], qa[1], fa, qb[0], qb[1], fb)
    print("case", fa, fb, M, N, K, flush=True)
    check_gemm(_host_c(_run(mx, qa, fa, qb, fb, False), False), C, S, False)


def test_ldc_and_zero_k(mx):
    import torch
    rng = np.random.default_rng(3)
    qa, qb = _rand_operand(rng, 70, 128, "e5m2"), _rand_operand(rng, 90, 128, "e4m3")
    C, S = oracle.gemm(qa[0], qa[1], "e5m2", qb[0], qb[1], "e4m3")
    big = torch.full((70, 128), 7.0, dtype=torch.float32, device="cuda")
    out = big[:, 10:100]
    _run(mx, qa, "e5m2", qb, "e4m3", False, out=out)
    h = to_host(big)
    check_gemm(h[:, 10:100].astype(np.float64), C, S, False)
    assert np.all(h[:, :10] == 7.0) and np.all(h[:, 100:] == 7.0)
    # K = 0: C = 0
    z = mx.gemm(torch.empty(5, 0, dtype=torch.uint8, device="cuda"), torch.empty(5, 0, dtype=torch.uint8, device="cuda"),
                "e4m3", torch.empty(6, 0, dtype=torch.uint8, device="cuda"),
                torch.empty(6, 0, dtype=torch.uint8, device="cuda"), "e4m3", out_dtype=torch.float32)
    assert np.all(to_host(z) == 0)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e2m1", "e2m1"), ("e5m2", "e4m3"), ("e4m3", "e2m1")])
@pytest.mark.parametrize("K", [352, 512, 1024])
def test_zero_and_nan_blocks(mx, fa, fb, K):
    """an all-zero block contributes exactly 0; an E8M0 NaN scale (0xFF) in row m of A
    makes row m of C NaN, and one in row n of B makes column n NaN (K = 352: the
    general kernels; K = 512 and 1024: the pipelined ones, with the NaN block in the
    first and in a later scale slot)"""
    rng = np.random.default_rng(8 + K + FMTS.index(fa) * 3 + FMTS.index(fb))
    M, N = 300, 272
    qa, qb = _rand_operand(rng, M, K, fa), _rand_operand(rng, N, K, fb)
    qa[0][3] = 0
    qa[1][3] = 0
    C, S = oracle.gemm(qa[0], qa[1], fa, qb[0], qb[1], fb)
    print("case", fa, fb, K, flush=True)
    for bf16 in (False, True):
        c = _host_c(_run(mx, qa, fa, qb, fb, bf16), bf16)
        assert np.all(c[3] == 0)
        check_gemm(c, C, S, bf16)
    kb = K // 32
    qa[1][5, 2] = 0xFF               # row 5 of A, block 2
    qa[1][261, kb - 1] = 0xFF        # a row of the second tile row, last block
    qb[1][7, kb // 2 + 1] = 0xFF     # row 7 of B (column 7 of C), a middle block
    qb[1][270, 0] = 0xFF             # a column of the second tile column, block 0
    C, S = oracle.gemm(qa[0], qa[1], fa, qb[0], qb[1], fb)
    nan_rows, nan_cols = [5, 261], [7, 270]
    for bf16 in (False, True):
        c = _host_c(_run(mx, qa, fa, qb, fb, bf16), bf16)
        assert np.all(np.isnan(c[nan_rows])), "NaN scale in A: row not NaN"
        assert np.all(np.isnan(c[:, nan_cols])), "NaN scale in B: column not NaN"
        keep_r = np.setdiff1d(np.arange(M), nan_rows)
        keep_c = np.setdiff1d(np.arange(N), nan_cols)
        sub = np.ix_(keep_r, keep_c)
        check_gemm(c[sub], C[sub], S[sub], bf16)


@pytest.mark.parametrize("M,N", [(300, 200), (257, 511), (40, 600)])
@pytest.mark.parametrize("bf16", [False, True])
def test_fp4_pipelined_tails(mx, M, N, bf16):
    """E2M1 x E2M1 with K % 512 == 0 (the pipelined kernel) and M, N not multiples
    of the 256 x 256 tile: rows past the edge read zeros through the buffer range
    and the LDS-staged epilogue masks its stores; every element checked"""
    rng = np.random.default_rng(M * 7 + N)
    K = 1024
    qa, qb = _rand_operand(rng, M, K, "e2m1"), _rand_operand(rng, N, K, "e2m1")
    C, S = oracle.gemm(qa[0], qa[1], "e2m1", qb[0], qb[1], "e2m1")
    print("case", M, N, K, "bf16" if bf16 else "f32", flush=True)
    check_gemm(_host_c(_run(mx, qa, "e2m1", qb, "e2m1", bf16), bf16), C, S, bf16)


def test_fp4_pipelined_tails_benchmark_shape(mx):
    """the benchmark's FP4 tail case: the gate/up operands cut to 8000 x 28000 x 4096
    (M and N ragged against the 256 x 256 tile), bf16 out; every row of the last,
    partial tile row and a seeded sample of the others, against all N columns"""
    cfg = workloads.config(2)
    M, N = 8000, 28000
    qa = tuple(t[:M] for t in _oracle_operands(cfg, "qX"))
    qb = tuple(t[:N] for t in _oracle_operands(cfg, "qW"))
    c = _host_c(_run(mx, qa, "e2m1", qb, "e2m1", True), True)
    rng = np.random.default_rng(8000)
    rows = np.unique(np.concatenate([np.arange(7936, M), rng.choice(7936, 448, replace=False)]))
    worst = 0.0
    for r0 in range(0, rows.size, 128):
        rr = rows[r0:r0 + 128]
        C, S = oracle.gemm(qa[0], qa[1], "e2m1", qb[0], qb[1], "e2m1", rows=rr)
        worst = max(worst, check_gemm(c[rr], C, S, True))
        print("rows %d of %d checked" % (min(r0 + 128, rows.size), rows.size), flush=True)
    print("max |err|/S", worst, flush=True)


FULL = [(1, "Y", True), (2, "Y", True), (3, "dW", False)]


@pytest.mark.parametrize("ci,gname,bf16", FULL)
def test_full_size_every_element(mx, ci, gname, bf16):
    """full-size GEMM launched as the benchmark launches it, every element of C
    against the oracle (computed in chunks of 2048 rows of A)"""
    cfg = workloads.config(ci)
    g = [x for x in cfg.gemms if x.name == gname][0]
    print("case", cfg.name, g.name, g.M, g.N, g.K, flush=True)
    qa_spec, qb_spec = cfg.quant(g.a), cfg.quant(g.b)
    qa, qb = _oracle_operands(cfg, g.a), _oracle_operands(cfg, g.b)
    c = _host_c(_run(mx, qa, qa_spec.fmt, qb, qb_spec.fmt, bf16), bf16)
    worst = 0.0
    for r0 in range(0, g.M, 2048):
        rows = np.arange(r0, min(g.M, r0 + 2048))
        C, S = oracle.gemm(qa[0], qa[1], qa_spec.fmt, qb[0], qb[1], qb_spec.fmt, rows=rows)
        worst = max(worst, check_gemm(c[rows], C, S, bf16))
        print("rows %d..%d checked" % (rows[0], rows[-1]), flush=True)
    print("max |err|/S", worst, flush=True)


def _random_codes(rng, rows, K, fmt):
    if fmt == "e2m1":
        c = rng.integers(0, 256, (rows, K // 2)).astype(np.uint8)
    else:
        c = rng.integers(0, 256, (rows, K)).astype(np.uint8)
        bad = (c & 0x7F) == 0x7F if fmt == "e4m3" else (c & 0x7C) == 0x7C
        c[bad] = 0x38
    return c


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e5m2")])
@pytest.mark.parametrize("K", [512, 1536, 2560])
def test_carrier_zero_stages_reference_scales(mx, fa, fb, K):
    """the FP8 carrier rebases each block's E8M0 byte on its row's largest one,
    R; at these K its loop runs stages past the end of K, which hold zero codes
    and zero scale bytes and must add exactly 0 for every R (with R = 128 a zero
    byte once rebased to an Inf scale, and 0 * Inf put NaN across the row).
    Rows' R cycle through 120..136; the other blocks lie up to 40 binades below."""
    rng = np.random.default_rng(K + 7 * FMTS.index(fa) + FMTS.index(fb))
    M, N = 256, 256
    ca, cb = _random_codes(rng, M, K, fa), _random_codes(rng, N, K, fb)
    kb = K // 32

    def scales(rows, R):
        s = (R[:, None] - rng.integers(0, 41, (rows, kb))).astype(np.uint8)
        s[np.arange(rows), rng.integers(0, kb, rows)] = R  # each row reaches its R
        return s

    sa = scales(M, 120 + np.arange(M) % 17)
    sb = scales(N, 120 + (3 * np.arange(N)) % 17)
    assert (sa.max(axis=1) == 128).any() and (sb.max(axis=1) == 128).any()
    C, S = oracle.gemm(ca, sa, fa, cb, sb, fb)
    for bf16 in (False, True):
        c = _host_c(_run(mx, (ca, sa), fa, (cb, sb), fb, bf16), bf16)
        assert not np.isnan(c).any(), "NaN in C"
        check_gemm(c, C, S, bf16)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e2m1"), ("e2m1", "e5m2"),
                                   ("e2m1", "e2m1")])
@pytest.mark.parametrize("spread", ["narrow", "full", "pathological"])
def test_scale_spreads(mx, fa, fb, spread):
    """codes and E8M0 scales drawn directly: narrow spreads (carrier fast path),
    spreads of up to 90 binades per row (exact per-block path), and rows whose
    only contributions come from blocks 2^100 below the row's largest scale"""
    rng = np.random.default_rng(["narrow", "full", "pathological"].index(spread) * 10 + FMTS.index(fa))
    M, N, K = 288, 320, 512
    ca, cb = _random_codes(rng, M, K, fa), _random_codes(rng, N, K, fb)
    if spread == "narrow":
        sa = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
        sb = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    elif spread == "full":
        # per-row spreads up to 90 binades (exact per-block path) while every
        # result stays inside the fp32 normal range the output can hold
        sa = rng.integers(80, 171, (M, K // 32)).astype(np.uint8)
        sb = rng.integers(80, 171, (N, K // 32)).astype(np.uint8)
    else:
        sa = rng.integers(120, 135, (M, K // 32)).astype(np.uint8)
        sb = rng.integers(120, 135, (N, K // 32)).astype(np.uint8)
        sa[:, 0] = 230                      # one huge block per A row ...
        cbz = cb.copy()
        nb = 16 if fb == "e2m1" else 32
        cbz[:, :nb] = 0                     # ... where every B column is zero
        cb = cbz
        sa[:, 1:] = rng.integers(10, 30, (M, K // 32 - 1))   # the rest ~2^-100 smaller
    C, S = oracle.gemm(ca, sa, fa, cb, sb, fb)
    assert np.all(np.isfinite(C))
    for bf16 in (False, True):
        c = _host_c(_run(mx, (ca, sa), fa, (cb, sb), fb, bf16), bf16)
        r = check_gemm(c, C, S, bf16)
        print(spread, fa, fb, "bf16" if bf16 else "f32", "max |err|/S", r)


@pytest.mark.parametrize("fa,fb", [("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e2m1")])
@pytest.mark.parametrize("case", ["zero_blocks", "zero_blocks_high_R", "tiny_blocks"])
def test_carrier_blocks_under_scale_zero(mx, fa, fb, case):
    """blocks whose E8M0 byte is 0 in rows whose other blocks lie 100+ binades
    higher (pipelined carrier, K = 1024).  All-zero blocks (codes of either
    sign) add exactly 0 and leave their tile on the fast path while the row's
    largest byte R <= 127; with R up to 135 the tile must take the exact
    per-block kernel (a rebased zero byte would borrow from its neighbours);
    a block of tiny nonzero values under byte 0 must take it too."""
    rng = np.random.default_rng(["zero_blocks", "zero_blocks_high_R", "tiny_blocks"].index(case) * 10
                                + FMTS.index(fa) + 3 * FMTS.index(fb))
    M, N, K = 300, 272, 1024
    kb = K // 32
    ca, cb = _random_codes(rng, M, K, fa), _random_codes(rng, N, K, fb)
    hi = 136 if case == "zero_blocks_high_R" else 128
    sa = rng.integers(hi - 30, hi, (M, kb)).astype(np.uint8)
    sb = rng.integers(hi - 30, hi, (N, kb)).astype(np.uint8)

    def clear(c, s, rows, blocks, fmt):
        nb = 16 if fmt == "e2m1" else 32
        neg = 0x88 if fmt == "e2m1" else 0x80
        for r, b in zip(rows, blocks):
            s[r, b] = 0
            c[r, b * nb:(b + 1) * nb] = neg if r % 3 == 0 else 0  # negative zeros in some rows

    rows_a = np.arange(0, M, 2)                      # every other row of A: one zero block
    clear(ca, sa, rows_a, rng.integers(0, kb, rows_a.size), fa)
    rows_b = np.arange(1, N, 5)
    clear(cb, sb, rows_b, rng.integers(0, kb, rows_b.size), fb)
    if case == "tiny_blocks":                        # a few byte-0 blocks keep nonzero codes
        for r in (4, 130, 262):
            b = int(rng.integers(0, kb))
            sa[r, b] = 0
    C, S = oracle.gemm(ca, sa, fa, cb, sb, fb)
    print("case", case, fa, fb, flush=True)
    for bf16 in (False, True):
        c = _host_c(_run(mx, (ca, sa), fa, (cb, sb), fb, bf16), bf16)
        assert not np.isnan(c).any(), "NaN in C"
        r = check_gemm(c, C, S, bf16)
        print(case, fa, fb, "bf16" if bf16 else "f32", "max |err|/S", r, flush=True)
