"""One GPU's share of an FSDP2 MXFP8 weight all-gather (MindSpeed-LLM FSDP2
page: weights sharded with shard_by_dim_0, all-gathered as MXFP8 codes and
E8M0 scales instead of bf16), and the strided operands that make the
gathered buffer a GEMM operand without a copy.

A rank quantizes only its slab of weight rows (dim 0 = N_out) into one
payload buffer of rows [codes | scales] (mx_quantize_strided).  K blocks
never cross rows, so the ranks' payloads concatenated in rank order -- what an
all-gather of one buffer per rank delivers -- hold exactly the codes and
scales of the whole weight, and mx_gemm_strided reads them in place."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import check_gemm, to_dev_bf16, to_dev_u8, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_block_amax_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
@pytest.mark.parametrize("ranks", [8, 7])
def test_payload_gathers_to_the_full_form(mx, fmt, ranks):
    import torch
    cfg = workloads.config(1)                    # Llama-3.1-8B QKV: W [6144 x 4096], X [8192 x 4096]
    w = workloads.draw_tensor(cfg, "W")
    wd = to_dev_bf16(w)
    n, K = w.shape
    bounds = np.linspace(0, n, ranks + 1).astype(int)   # 7 ranks: slabs not on tile boundaries
    payloads = [mx.fsdp_payload(wd[bounds[r]:bounds[r + 1]], fmt) for r in range(ranks)]
    width = mx.payload_width(K, fmt)
    assert width == mx.code_cols(K, fmt) + K // 32      # K % 512 == 0: no padding
    assert all(p.shape == (bounds[r + 1] - bounds[r], width) for r, p in enumerate(payloads))
    gathered = torch.cat(payloads)               # the all-gather of one buffer per rank, in rank order
    codes, scales = mx.payload_views(gathered, K, fmt)
    full = oracle.quantize(w, fmt)
    assert np.array_equal(to_host(codes), full[0]) and np.array_equal(to_host(scales), full[1])
    print("payload %s, %d ranks: %.4f bytes per element (bf16: 2)" % (fmt, ranks, width / K), flush=True)

    # the gathered payload is the GEMM's B operand as is (Fprop Y = X W^T): sampled rows
    # against the oracle, and every element against the dense operand's result
    x = workloads.draw_tensor(cfg, "X", rows=(0, 512))
    qx = mx.quantize(to_dev_bf16(x), fmt)
    for out_dtype, bf16 in ((torch.float32, False), (torch.bfloat16, True)):
        y = mx.gemm(qx[0], qx[1], fmt, codes, scales, fmt, out_dtype=out_dtype)
        y_dense = mx.gemm(qx[0], qx[1], fmt, to_dev_u8(full[0]), to_dev_u8(full[1]), fmt, out_dtype=out_dtype)
        assert torch.equal(y.view(torch.int16) if bf16 else y.view(torch.int32),
                           y_dense.view(torch.int16) if bf16 else y_dense.view(torch.int32))
        ox = oracle.quantize(x, fmt)
        rows = np.array([0, 17, 128, 255, 300, 511])
        C, S = oracle.gemm(ox[0], ox[1], fmt, full[0], full[1], fmt, rows=rows)
        got = to_host(y)[rows]
        got = workloads.bf16_bits_to_f32(got).astype(np.float64) if bf16 else got.astype(np.float64)
        check_gemm(got, C, S, bf16)


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_dense_slabs_gather_to_the_full_form(mx, fmt):
    """the same with separate codes and scales per rank (mx_quantize on a row range)"""
    import torch
    cfg = workloads.config(1)
    w = workloads.draw_tensor(cfg, "W")
    wd = to_dev_bf16(w)
    bounds = np.linspace(0, w.shape[0], 8).astype(int)
    parts = [mx.quantize(wd[bounds[r]:bounds[r + 1]], fmt) for r in range(7)]
    full = oracle.quantize(w, fmt)
    assert np.array_equal(to_host(torch.cat([p[0] for p in parts])), full[0])
    assert np.array_equal(to_host(torch.cat([p[1] for p in parts])), full[1])


def _operand(rng, rows, K, fmt):
    import torch
    v = (rng.standard_t(4, (rows, K)) * np.exp2(rng.integers(-6, 6, (rows, K // 32))).repeat(32, 1)).astype(np.float32)
    bits = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return oracle.quantize(bits, fmt)


def _embed(q, pad_codes, pad_scales):
    """codes and scales of q placed in buffers with padded rows (row-strided views)"""
    import torch
    c, s = q
    bc = torch.full((c.shape[0], c.shape[1] + pad_codes), 0x5A, dtype=torch.uint8, device="cuda")
    bs = torch.full((s.shape[0], s.shape[1] + pad_scales), 0x7F, dtype=torch.uint8, device="cuda")
    bc[:, :c.shape[1]] = to_dev_u8(c)
    bs[:, :s.shape[1]] = to_dev_u8(s)
    return bc[:, :c.shape[1]], bs[:, :s.shape[1]]


@pytest.mark.parametrize("fa,fb", [("e2m1", "e2m1"), ("e4m3", "e4m3"), ("e5m2", "e4m3"), ("e4m3", "e2m1")])
@pytest.mark.parametrize("K,pads", [(1024, (32, 16, 48, 32)),   # aligned strides: the pipelined kernel
                                    (1024, (16, 3, 32, 4)),     # scale strides not 16-byte multiples: general kernels
                                    (352, (16, 4, 16, 4))])     # K % 512 != 0: the general kernels
def test_gemm_strided_operands(mx, fa, fb, K, pads):
    """row-strided codes and scales (padding bytes hold garbage) give the dense
    operands' result within the tolerance, bit for bit when the strides keep the
    dense call's kernel; M and N ragged against the tile"""
    import torch
    rng = np.random.default_rng(K + sum(pads))
    M, N = 300, 520
    qa, qb = _operand(rng, M, K, fa), _operand(rng, N, K, fb)
    C, S = oracle.gemm(qa[0], qa[1], fa, qb[0], qb[1], fb)
    a, b = _embed(qa, pads[0], pads[1]), _embed(qb, pads[2], pads[3])
    assert not a[0].is_contiguous() and not b[1].is_contiguous()
    print("case", fa, fb, K, pads, flush=True)
    same_kernel = all(p % 16 == 0 for p in pads)
    for out_dtype, bf16 in ((torch.float32, False), (torch.bfloat16, True)):
        y = mx.gemm(a[0], a[1], fa, b[0], b[1], fb, out_dtype=out_dtype)
        got = to_host(y)
        got = workloads.bf16_bits_to_f32(got).astype(np.float64) if bf16 else got.astype(np.float64)
        check_gemm(got, C, S, bf16)
        if same_kernel or K % 512:
            y_dense = mx.gemm(to_dev_u8(qa[0]), to_dev_u8(qa[1]), fa, to_dev_u8(qb[0]), to_dev_u8(qb[1]), fb,
                              out_dtype=out_dtype)
            assert np.array_equal(to_host(y).view(np.uint8), to_host(y_dense).view(np.uint8))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "e2m1"])
def test_quantize_strided_outputs(mx, fmt):
    """row-mode codes and scales written with row strides into padded buffers
    equal the dense call's; the padding is left untouched"""
    import torch
    rng = np.random.default_rng(5)
    rows, cols = 130, 640
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, (rows, 1)))).astype(np.float32)
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    dense = mx.quantize(xd, fmt)
    cb = mx.code_cols(cols, fmt)
    for pc, ps in ((16, 12), (3, 1)):
        bc = torch.full((rows, cb + pc), 0xA5, dtype=torch.uint8, device="cuda")
        bs = torch.full((rows, cols // 32 + ps), 0xA5, dtype=torch.uint8, device="cuda")
        mx.quantize(xd, fmt, out=(bc[:, :cb], bs[:, :cols // 32]))
        assert torch.equal(bc[:, :cb], dense[0]) and torch.equal(bs[:, :cols // 32], dense[1])
        assert bool((bc[:, cb:] == 0xA5).all()) and bool((bs[:, cols // 32:] == 0xA5).all())
