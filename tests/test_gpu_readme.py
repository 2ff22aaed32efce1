"""The README's usage example runs as printed and agrees with the oracle.

The Python block of README.md (one gate/up linear layer in the MXFP4 recipe:
Fprop, Dgrad through the transposed weight, rotated Wgrad) is executed as it
stands.  Its quantized operands must equal the oracle's quantization of the
same bf16 inputs byte for byte, and its three products must be within the
GEMM tolerance on sampled rows (first and last included) against all columns.
"""
import os
import re

import numpy as np
import pytest

import oracle
import workloads
from helpers import check_gemm, to_host

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def readme_example() -> str:
    with open(os.path.join(ROOT, "README.md")) as f:
        blocks = re.findall(r"```python\n(.*?)```", f.read(), re.S)
    assert len(blocks) == 1, "README.md should hold one Python example"
    return blocks[0]


def test_readme_example_matches_oracle():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.manual_seed(0)
    ns = {}
    exec(compile(readme_example(), "README.md", "exec"), ns)
    torch.cuda.synchronize()
    bits = {k: to_host(ns[k]) for k in ("x", "w", "dy")}

    def same(gpu, ref, what):
        for part, g, r in (("codes", gpu[0], ref[0]), ("scales", gpu[1], ref[1])):
            assert np.array_equal(to_host(g), r), "%s %s differ from the oracle" % (what, part)

    ox, ow = oracle.quantize(bits["x"], "e2m1"), oracle.quantize(bits["w"], "e2m1")
    same(ns["qx"], ox, "qx")
    same(ns["qw"], ow, "qw")
    ody, owt = oracle.quantize(bits["dy"], "e2m1"), oracle.quantize_transpose(bits["w"], "e2m1")
    same(ns["qdy"], ody, "qdy")
    same(ns["qwt"], owt, "qwt")
    odyh, oxh = oracle.hadamard32_quantize(bits["dy"], "e2m1", 0), oracle.hadamard32_quantize(bits["x"], "e2m1", 0)
    same(ns["qdy_h"], odyh, "qdy_h")
    same(ns["qx_h"], oxh, "qx_h")

    rng = np.random.default_rng(1)
    for name, a, b, bf16 in (("y", ox, ow, True), ("dx", ody, owt, True), ("dw", odyh, oxh, False)):
        got = to_host(ns[name])
        m = got.shape[0]
        rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 6, replace=False)]))
        C, S = oracle.gemm(a[0], a[1], "e2m1", b[0], b[1], "e2m1", rows=rows)
        g = workloads.bf16_bits_to_f32(got[rows]).astype(np.float64) if bf16 else got[rows].astype(np.float64)
        r = check_gemm(g, C, S, bf16)
        print(name, "max |err|/S on rows", rows.tolist(), r, flush=True)
