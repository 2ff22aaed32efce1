"""GPU parity of one whole Llama-3.1-8B gate+up linear layer in the MXFP4 recipe
(FP4-training article on hzrcw.cc, section 02: the forward, activation-gradient
and weight-gradient GEMMs all in MXFP4, the weight gradient's operands rotated
by the fixed block-Hadamard transform), at full size, with every operand made
by the dual-direction quantizer the way a training step would make it:

  X  [8192 x 4096]  -> row form (Fprop A)  + rotated transposed form (Wgrad B)
  W  [28672 x 4096] -> row form (Fprop B)  + transposed form (Dgrad B)
  dY [8192 x 28672] -> row form (Dgrad A)  + rotated transposed form (Wgrad A)

  Fprop  Y  = X W^T   [8192 x 28672], K = 4096,  bf16 out
  Dgrad  dX = dY W    [8192 x 4096],  K = 28672, bf16 out
  Wgrad  dW = dY^T X  [28672 x 4096], K = 8192,  fp32 out

Both forms of every tensor are compared with the oracle on every code and
scale; each GEMM is checked on 512 seeded rows against all columns."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import check_gemm, to_dev_bf16, to_host

pytestmark = pytest.mark.gpu
CFG = workloads.config(5)
MASK = 0


@pytest.fixture(scope="module")
def layer():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_block_amax_amd as mx
    mx.lib()
    ops, ref = {}, {}
    for src, q_row, q_t in workloads.LAYER_DUALS:
        bits = workloads.draw_tensor(CFG, src)
        qr, qt = CFG.quant(q_row), CFG.quant(q_t)
        rotate = qt.kind == "hadamard"
        print("dual quantize %s %s" % (src, bits.shape), flush=True)
        cr, sr, ct, st = mx.quantize_dual(to_dev_bf16(bits), qr.fmt, qt.fmt, rotate, MASK)
        ops[q_row], ops[q_t] = (cr, sr), (ct, st)
        ref[q_row] = oracle.quantize(bits, qr.fmt)
        ref[q_t] = (oracle.hadamard32_quantize(bits, qt.fmt, MASK) if rotate
                    else oracle.quantize_transpose(bits, qt.fmt))
    return mx, ops, ref


@pytest.mark.parametrize("qname", [q.name for q in CFG.quants])
def test_layer_operands_every_code_and_scale(layer, qname):
    _, ops, ref = layer
    for part in (0, 1):
        got = to_host(ops[qname][part])
        bad = np.nonzero(got != ref[qname][part])
        assert bad[0].size == 0, "%s %s: %d mismatches" % (qname, ("codes", "scales")[part], bad[0].size)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("gname", [g.name for g in CFG.gemms])
def test_layer_gemm_sampled_rows(layer, gname):
    import torch
    mx, ops, ref = layer
    g = [x for x in CFG.gemms if x.name == gname][0]
    qa, qb = CFG.quant(g.a), CFG.quant(g.b)
    bf16 = g.out == "bf16"
    print("case", CFG.name, g.name, g.M, g.N, g.K, flush=True)
    c = mx.gemm(ops[g.a][0], ops[g.a][1], qa.fmt, ops[g.b][0], ops[g.b][1], qb.fmt,
                out_dtype=torch.bfloat16 if bf16 else torch.float32)
    rng = np.random.default_rng([x.name for x in CFG.gemms].index(gname) + 50)
    rows = np.unique(np.concatenate([[0, g.M - 1], rng.choice(g.M, 510, replace=False)]))
    got = to_host(c[torch.from_numpy(rows).cuda()])
    got = workloads.bf16_bits_to_f32(got).astype(np.float64) if bf16 else got.astype(np.float64)
    ra, rb = ref[g.a], ref[g.b]
    chunk = max(256, (1 << 29) // (8 * g.K) // 256 * 256)
    worst = 0.0
    for n0 in range(0, g.N, chunk):
        n1 = min(g.N, n0 + chunk)
        C, S = oracle.gemm(ra[0][rows], ra[1][rows], qa.fmt, rb[0][n0:n1], rb[1][n0:n1], qb.fmt)
        worst = max(worst, check_gemm(got[:, n0:n1], C, S, bf16))
    print("max |err|/S", worst, flush=True)


def _to_panels(codes: np.ndarray) -> np.ndarray:
    """row-major codes [R x Kbytes] -> K-panel layout [Kbytes/128 x R x 128]"""
    r, kb = codes.shape
    return np.ascontiguousarray(codes.reshape(r, kb // 128, 128).transpose(1, 0, 2))


@pytest.mark.timeout(600)
def test_layer_in_k_panels(layer):
    """the same layer with every operand in the K-panel layout (mx_quantize_dual_panels):
    both forms of every tensor equal to the oracle's codes cut into panels, byte for
    byte, and each GEMM through mx_gemm_layout bit-identical to mx_gemm on the
    row-major operands above"""
    import torch
    mx, ops, ref = layer
    pops = {}
    for src, q_row, q_t in workloads.LAYER_DUALS:
        bits = workloads.draw_tensor(CFG, src)
        qr, qt = CFG.quant(q_row), CFG.quant(q_t)
        print("dual quantize in panels %s %s" % (src, bits.shape), flush=True)
        cr, sr, ct, st = mx.quantize_dual(to_dev_bf16(bits), qr.fmt, qt.fmt, qt.kind == "hadamard", MASK,
                                          layout="panels")
        pops[q_row], pops[q_t] = (cr, sr), (ct, st)
        for q, (c, s) in ((q_row, (cr, sr)), (q_t, (ct, st))):
            assert np.array_equal(to_host(s), ref[q][1]), "%s scales" % q
            assert np.array_equal(to_host(c), _to_panels(ref[q][0])), "%s codes" % q
    for g in CFG.gemms:
        qa, qb = CFG.quant(g.a), CFG.quant(g.b)
        dt = torch.bfloat16 if g.out == "bf16" else torch.float32
        print("case", g.name, g.M, g.N, g.K, flush=True)
        c = mx.gemm(pops[g.a][0], pops[g.a][1], qa.fmt, pops[g.b][0], pops[g.b][1], qb.fmt, out_dtype=dt)
        d = mx.gemm(ops[g.a][0], ops[g.a][1], qa.fmt, ops[g.b][0], ops[g.b][1], qb.fmt, out_dtype=dt)
        iv = torch.int16 if dt == torch.bfloat16 else torch.int32
        assert torch.equal(c.view(iv), d.view(iv)), g.name
        del c, d
