"""GPU parity of the stochastic-rounding quantizer (mx_quantize_transpose_sr)
against the oracle: codes and scales bit-exact for the same seed.

The kernel computes its own Philox4x32-10 words; the oracle computes them
independently from the generator's definition.  Cases: the small MXFP8 case
and the weight-gradient tensors at full size, with and without the rotation,
two seeds (one with a non-zero high key word); the edge suite; every finite
bf16 at every scale; ragged, strided and unaligned layouts; repeatability.
"""
import numpy as np
import pytest

import oracle
import workloads
from helpers import to_dev_bf16, to_host
from test_gpu_quantize import FMTS, _cmp, _rand_bits, edge_cols, exhaustive_blocks

pytestmark = pytest.mark.gpu
SEEDS = (0, 0xDEADBEEFCAFEF00D)


@pytest.fixture(scope="module")
def mx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_block_amax_amd as m
    m.lib()
    return m


SR_CASES = [(0, "B", "e4m3", False, 0, SEEDS[0]), (0, "B", "e2m1", True, 0x9E3779B9, SEEDS[1]),
            (0, "B", "e5m2", True, 0, SEEDS[1]),
            (3, "dY", "e2m1", True, 0, SEEDS[0]), (3, "X", "e2m1", True, 0, SEEDS[1]),
            (3, "dY", "e2m1", False, 0, SEEDS[1])]


@pytest.mark.parametrize("ci,name,fmt,rotate,mask,seed", SR_CASES)
def test_sr_workloads(mx, ci, name, fmt, rotate, mask, seed):
    cfg = workloads.config(ci)
    x = workloads.draw_tensor(cfg, name)
    print("case", cfg.name, name, fmt, rotate, hex(mask), hex(seed), x.shape, flush=True)
    got = mx.quantize_transpose_sr(to_dev_bf16(x), fmt, seed, rotate, mask)
    _cmp(got, oracle.quantize_transpose_sr(x, fmt, seed, rotate, mask), "%s/%s SR" % (cfg.name, name))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rotate", [False, True])
def test_sr_edge_suite(mx, fmt, rotate):
    x = edge_cols()
    for seed in SEEDS:
        got = mx.quantize_transpose_sr(to_dev_bf16(x), fmt, seed, rotate, 0x9E3779B9)
        _cmp(got, oracle.quantize_transpose_sr(x, fmt, seed, rotate, 0x9E3779B9), "edge SR")


@pytest.mark.parametrize("fmt", FMTS)
def test_sr_every_bf16_at_every_scale(mx, fmt):
    """every finite bf16 value at every reachable scale exponent, rounded
    stochastically (the rule's every binade, subnormal range and saturation)"""
    xt = np.ascontiguousarray(exhaustive_blocks(fmt).T)
    got = mx.quantize_transpose_sr(to_dev_bf16(xt), fmt, SEEDS[1])
    _cmp(got, oracle.quantize_transpose_sr(xt, fmt, SEEDS[1]), "SR, every bf16 x every e")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("rows,cols,extra", [(32, 1, 0), (64, 37, 0), (96, 255, 0), (160, 258, 0), (224, 300, 2)])
def test_sr_ragged_strided(mx, fmt, rotate, rows, cols, extra):
    full = _rand_bits(rows, cols + extra, rows * 5 + cols)
    xd = to_dev_bf16(full)[:, :cols]
    x = np.ascontiguousarray(full[:, :cols])
    _cmp(mx.quantize_transpose_sr(xd, fmt, 7, rotate, 0x12345678),
         oracle.quantize_transpose_sr(x, fmt, 7, rotate, 0x12345678), "ragged SR")


def test_sr_unaligned_codes(mx):
    import torch
    x = _rand_bits(64, 128, 98)
    cbuf = torch.empty(128 * 32 + 1, dtype=torch.uint8, device="cuda")
    codes = cbuf[1:].view(128, 32)
    scales = torch.empty(128, 2, dtype=torch.uint8, device="cuda")
    mx.quantize_transpose_sr(to_dev_bf16(x), "e2m1", 3, True, 0, out=(codes, scales))
    _cmp((codes, scales), oracle.quantize_transpose_sr(x, "e2m1", 3, True, 0), "unaligned SR")


def test_sr_repeatable_and_seeded(mx):
    cfg = workloads.config(3)
    x = to_dev_bf16(workloads.draw_tensor(cfg, "dY", rows=(0, 512)))
    a = [to_host(t) for t in mx.quantize_transpose_sr(x, "e2m1", 5, True)]
    b = [to_host(t) for t in mx.quantize_transpose_sr(x, "e2m1", 5, True)]
    c = [to_host(t) for t in mx.quantize_transpose_sr(x, "e2m1", 6, True)]
    r = [to_host(t) for t in mx.hadamard32_quantize(x, "e2m1", 0)]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0])
    assert np.array_equal(a[1], r[1]), "scales are the round-to-nearest quantizer's"
