"""GPU parity on the Llama-3.1-70B linear-layer set at full size: all nine
GEMMs (Fprop, Dgrad through the transposed weight, and the rotated FP4
down-projection Wgrad), with E4M3 activations and weights and E5M2 output
gradients, as the configuration lists them.

Each case quantizes both full operands on the GPU and multiplies them as the
library would in training.  The oracle quantizes the same full operands on
its own; every code and every scale must match bit for bit (the nine GEMMs'
eighteen operands are the configuration's eighteen quantize calls).  C is
then checked on 512 seeded rows (first and last row included) against every
column, within |err| <= 1e-5 * sum |a*b| (plus half a bf16 ulp for bf16
output); the oracle's fp64 product runs over column chunks of B so that its
dequantized operand stays bounded in host memory.  Checking all 8192 rows of
the 32 TFLOP set takes the oracle minutes on many host cores, which is why C
is sampled by rows while the operands are compared in full.

Where the benchmark quantizes a GEMM's two operands in one pair launch (both
in one mode; rotated pairs in the K-panel layout), that launch runs too: its
outputs must equal the single calls' outputs above, byte for byte (cut into
panels where it writes panels), and the GEMM is then run on them, as the
benchmark runs it."""
import numpy as np
import pytest

import bench
import oracle
import workloads
from helpers import check_gemm, to_dev_bf16, to_host

pytestmark = pytest.mark.gpu
CFG = workloads.config(4)
SAMPLE_ROWS = 512
B_CHUNK_BYTES = 1 << 29  # dequantized float64 B per oracle call


@pytest.fixture(scope="module")
def mx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_block_amax_amd as m
    m.lib()
    return m


_tensors = {}


def tensor(name):
    """full source tensor, generated once per module (host bits, device copy)"""
    if name not in _tensors:
        while len(_tensors) >= 3:  # keep host and device memory bounded
            _tensors.pop(next(iter(_tensors)))
        bits = workloads.draw_tensor(CFG, name)
        _tensors[name] = (bits, to_dev_bf16(bits))
    return _tensors[name]


def gpu_quant(mx, q):
    _, dev = tensor(q.tensor)
    if q.kind == "row":
        return mx.quantize(dev, q.fmt)
    if q.kind == "transpose":
        return mx.quantize_transpose(dev, q.fmt)
    return mx.hadamard32_quantize(dev, q.fmt, q.sign_mask)


def oracle_quant(q):
    bits, _ = tensor(q.tensor)
    if q.kind == "row":
        return oracle.quantize(bits, q.fmt)
    if q.kind == "transpose":
        return oracle.quantize_transpose(bits, q.fmt)
    return oracle.hadamard32_quantize(bits, q.fmt, q.sign_mask)


def assert_operand_equal(name, gpu, ref):
    for part, g, r in (("codes", gpu[0], ref[0]), ("scales", gpu[1], ref[1])):
        g = to_host(g)
        assert g.shape == r.shape, (name, part, g.shape, r.shape)
        bad = np.nonzero(g != r)
        assert bad[0].size == 0, "%s %s differ from the oracle at %d places, first %s: gpu %#x oracle %#x" % (
            name, part, bad[0].size, (bad[0][0], bad[1][0]), g[bad[0][0], bad[1][0]], r[bad[0][0], bad[1][0]])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("gname", [g.name for g in CFG.gemms])
def test_70b_gemm(mx, gname):
    import torch
    g = [x for x in CFG.gemms if x.name == gname][0]
    qa, qb = CFG.quant(g.a), CFG.quant(g.b)
    print("case", CFG.name, g.name, g.M, g.N, g.K, qa.name, qa.fmt, qb.name, qb.fmt, flush=True)

    a_gpu = gpu_quant(mx, qa)
    a_ref = oracle_quant(qa)
    assert_operand_equal(qa.name, a_gpu, a_ref)
    print("operand %s: every code and scale equal" % qa.name, flush=True)
    b_gpu = gpu_quant(mx, qb)
    b_ref = oracle_quant(qb)
    assert_operand_equal(qb.name, b_gpu, b_ref)
    print("operand %s: every code and scale equal" % qb.name, flush=True)

    pair, panels = bench.pair_layout((qa, qb), (tensor(qa.tensor)[0].shape, tensor(qb.tensor)[0].shape))
    if pair:
        mode = qa.kind + ("_panels" if panels else "")
        pa, pb = mx.quantize_pair(mode, tensor(qa.tensor)[1], tensor(qb.tensor)[1], qa.fmt, qa.sign_mask)
        for got, single, name in ((pa, a_gpu, qa.name), (pb, b_gpu, qb.name)):
            want = single[0]
            if panels:  # row-major [R x Kbytes] -> [Kbytes/128 x R x 128]
                want = want.view(want.shape[0], want.shape[1] // 128, 128).permute(1, 0, 2).contiguous()
            assert torch.equal(got[0], want) and torch.equal(got[1], single[1]), "%s: pair launch" % name
        print("pair launch %s: both operands equal to the single calls" % mode, flush=True)
        a_gpu, b_gpu = pa, pb

    bf16 = g.out == "bf16"
    c = mx.gemm(a_gpu[0], a_gpu[1], qa.fmt, b_gpu[0], b_gpu[1], qb.fmt,
                out_dtype=torch.bfloat16 if bf16 else torch.float32)
    rng = np.random.default_rng([x.name for x in CFG.gemms].index(gname))
    rows = np.unique(np.concatenate([[0, g.M - 1], rng.choice(g.M, SAMPLE_ROWS - 2, replace=False)]))
    got = to_host(c[torch.from_numpy(rows).cuda()])
    del a_gpu, b_gpu, c
    got = workloads.bf16_bits_to_f32(got).astype(np.float64) if bf16 else got.astype(np.float64)

    chunk = max(256, B_CHUNK_BYTES // (8 * g.K) // 256 * 256)
    a_rows = (a_ref[0][rows], a_ref[1][rows])
    worst = 0.0
    for n0 in range(0, g.N, chunk):
        n1 = min(g.N, n0 + chunk)
        C, S = oracle.gemm(a_rows[0], a_rows[1], qa.fmt, b_ref[0][n0:n1], b_ref[1][n0:n1], qb.fmt)
        worst = max(worst, check_gemm(got[:, n0:n1], C, S, bf16))
        print("columns %d..%d of %d checked on %d rows" % (n0, n1 - 1, g.N, rows.size), flush=True)
    print("max |err|/S", worst, flush=True)
