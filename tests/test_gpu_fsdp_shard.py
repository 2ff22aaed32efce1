"""One GPU's share of an FSDP2 MXFP8 weight all-gather (MindSpeed-LLM FSDP2
page: weights sharded with shard_by_dim_0, all-gathered as MXFP8 codes and
E8M0 scales instead of bf16).

A rank quantizes only its slab of weight rows (dim 0 = N_out), with
mx_quantize on a row range of the weight (ldx = the full row).  K blocks
never cross rows, so the slabs' codes and scales, concatenated in rank order
(what the all-gather delivers), are bit-identical to quantizing the whole
weight, and mx_gemm consumes the gathered buffers directly."""
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
def test_sharded_quantize_gathers_to_the_full_form(mx, fmt, ranks):
    import torch
    cfg = workloads.config(1)                    # Llama-3.1-8B QKV: W [6144 x 4096], X [8192 x 4096]
    w = workloads.draw_tensor(cfg, "W")
    wd = to_dev_bf16(w)
    n = w.shape[0]
    bounds = np.linspace(0, n, ranks + 1).astype(int)   # 7 ranks: slabs not on tile boundaries
    parts = [mx.quantize(wd[bounds[r]:bounds[r + 1]], fmt) for r in range(ranks)]
    codes = torch.cat([p[0] for p in parts])     # the all-gather, in rank order
    scales = torch.cat([p[1] for p in parts])
    full = oracle.quantize(w, fmt)
    assert np.array_equal(to_host(codes), full[0]) and np.array_equal(to_host(scales), full[1])

    # the gathered payload feeds the GEMM as is (Fprop Y = X W^T), sampled rows against the oracle
    x = workloads.draw_tensor(cfg, "X", rows=(0, 256))
    qx = mx.quantize(to_dev_bf16(x), fmt)
    y = mx.gemm(qx[0], qx[1], fmt, codes, scales, fmt, out_dtype=torch.float32)
    ox = oracle.quantize(x, fmt)
    rows = np.array([0, 17, 128, 255])
    C, S = oracle.gemm(ox[0], ox[1], fmt, full[0], full[1], fmt, rows=rows)
    check_gemm(to_host(y)[rows].astype(np.float64), C, S, False)
