"""GPU parity on the Llama-3.1-70B linear-layer set at full size: all nine
GEMMs (Fprop, Dgrad through the transposed weight, and the rotated FP4
down-projection Wgrad), with E4M3 activations and weights and E5M2 output
gradients, as the configuration lists them.

Each case quantizes both full operands on the GPU and multiplies them as the
library would in training, then checks samples the oracle computes on its
own: quantized operand rows bit-exact, and 32 sampled rows x four random
256-column tiles of C within |err| <= 1e-5 * sum |a*b| (plus half a bf16 ulp
for bf16 output).
Row-mode operand rows are quantized rows of the source; transposed and
rotated operand rows are quantized columns of the source, so the oracle
needs only the sampled rows or columns."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import check_gemm, to_dev_bf16, to_host

pytestmark = pytest.mark.gpu
CFG = workloads.config(4)


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
        if len(_tensors) >= 4:  # keep host and device memory bounded
            _tensors.pop(next(iter(_tensors)))
        bits = workloads.draw_tensor(CFG, name)
        _tensors[name] = (bits, to_dev_bf16(bits))
    return _tensors[name]


def gpu_quant(mx, q):
    bits, dev = tensor(q.tensor)
    if q.kind == "row":
        return mx.quantize(dev, q.fmt)
    if q.kind == "transpose":
        return mx.quantize_transpose(dev, q.fmt)
    return mx.hadamard32_quantize(dev, q.fmt, q.sign_mask)


def oracle_rows(q, idx):
    """the oracle's quantization of operand rows idx only"""
    bits, _ = tensor(q.tensor)
    if q.kind == "row":
        return oracle.quantize(np.ascontiguousarray(bits[idx]), q.fmt)
    cols = np.ascontiguousarray(bits[:, idx])
    if q.kind == "transpose":
        return oracle.quantize_transpose(cols, q.fmt)
    return oracle.hadamard32_quantize(cols, q.fmt, q.sign_mask)


@pytest.mark.parametrize("gname", [g.name for g in CFG.gemms])
def test_70b_gemm_sampled(mx, gname):
    import torch
    g = [x for x in CFG.gemms if x.name == gname][0]
    qa, qb = CFG.quant(g.a), CFG.quant(g.b)
    print("case", CFG.name, g.name, g.M, g.N, g.K, qa.fmt, qb.fmt, flush=True)
    rng = np.random.default_rng([x.name for x in CFG.gemms].index(gname))
    rows = np.unique(np.concatenate([[0, g.M - 1], rng.integers(0, g.M, 30)]))
    tiles = np.sort(rng.choice(g.N // 256, 4, replace=False))  # four column tiles of C
    cols = np.concatenate([np.arange(t * 256, t * 256 + 256) for t in tiles])

    a_codes, a_scales = gpu_quant(mx, qa)
    b_codes, b_scales = gpu_quant(mx, qb)
    ora, orb = oracle_rows(qa, rows), oracle_rows(qb, cols)
    ri, ci = torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()
    assert np.array_equal(to_host(a_codes[ri]), ora[0]) and np.array_equal(to_host(a_scales[ri]), ora[1]), \
        "operand A rows differ from the oracle"
    assert np.array_equal(to_host(b_codes[ci]), orb[0]) and np.array_equal(to_host(b_scales[ci]), orb[1]), \
        "operand B rows differ from the oracle"

    bf16 = g.out == "bf16"
    c = mx.gemm(a_codes, a_scales, qa.fmt, b_codes, b_scales, qb.fmt,
                out_dtype=torch.bfloat16 if bf16 else torch.float32)
    got = to_host(c[ri][:, ci])
    del a_codes, a_scales, b_codes, b_scales, c
    got = workloads.bf16_bits_to_f32(got).astype(np.float64) if bf16 else got.astype(np.float64)
    C, S = oracle.gemm(ora[0], ora[1], qa.fmt, orb[0], orb[1], qb.fmt)
    r = check_gemm(got, C, S, bf16)
    print("max |err|/S", r, flush=True)
