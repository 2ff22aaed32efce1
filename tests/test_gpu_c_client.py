"""The C ABI from C: tests/c_client/mx_c_client.c (C99, built by build()
against include/mx.h and the in-tree libmx.so, with device memory and a
stream from the HIP runtime) runs the small MXFP8 case end to end -- A
[256 x 512] in row mode, B [512 x 256] stored as written in transposed mode,
both E4M3, then the GEMM with fp32 output -- and writes its results to
files.  Codes and scales must equal the oracle's byte for byte, and every
element of C must be within |err| <= 1e-5 * sum |a*b| of the oracle's
product.  The client also checks that a bad argument is rejected before any
launch."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads
from helpers import check_gemm

pytestmark = pytest.mark.gpu
CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "mx_c_client")


def test_c_client_small_case(tmp_path):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    assert os.path.exists(CLIENT), "build() builds the C client"
    cfg = workloads.config(0)
    a, b = workloads.draw_tensor(cfg, "A"), workloads.draw_tensor(cfg, "B")
    (M, K), (_, N) = a.shape, b.shape
    a.tofile(tmp_path / "a.bin")
    b.tofile(tmp_path / "b.bin")
    print("case", cfg.name, M, N, K, flush=True)
    r = subprocess.run([CLIENT, str(tmp_path), str(M), str(K), str(N)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")

    def rd(name, shape, dtype=np.uint8):
        return np.fromfile(tmp_path / name, dtype=dtype).reshape(shape)

    qa, qb = oracle.quantize(a, "e4m3"), oracle.quantize_transpose(b, "e4m3")
    assert np.array_equal(rd("qa_codes.bin", (M, K)), qa[0])
    assert np.array_equal(rd("qa_scales.bin", (M, K // 32)), qa[1])
    assert np.array_equal(rd("qb_codes.bin", (N, K)), qb[0])
    assert np.array_equal(rd("qb_scales.bin", (N, K // 32)), qb[1])
    C, S = oracle.gemm(qa[0], qa[1], "e4m3", qb[0], qb[1], "e4m3")
    r = check_gemm(rd("c.bin", (M, N), np.float32).astype(np.float64), C, S, False)
    print("max |err|/S", r, flush=True)
