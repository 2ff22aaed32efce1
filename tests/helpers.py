"""Shared helpers for the parity tests: inputs, device transfer, tolerances."""
from __future__ import annotations

import numpy as np

import workloads


def to_dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_dev_u8(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def to_host(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


def gemm_tolerance(c_ref: np.ndarray, s_abs: np.ndarray, bf16_out: bool) -> np.ndarray:
    """|err| bound per element: 1e-5 * sum|a*b| for the fp32 accumulator,
    plus half a bf16 ulp of the largest admissible fp32 value when the
    output is rounded to bf16."""
    tol = 1e-5 * s_abs
    if bf16_out:
        v = np.abs(c_ref) + tol
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
        e = np.maximum(e, -126)
        tol = tol + np.where(v > 0, np.ldexp(0.5, (e - 7).astype(np.int64)), 0.0)
    return tol


def check_gemm(c_gpu: np.ndarray, c_ref: np.ndarray, s_abs: np.ndarray, bf16_out: bool) -> float:
    """assert the bound element by element; return max |err| / S_abs"""
    err = np.abs(c_gpu.astype(np.float64) - c_ref)
    tol = gemm_tolerance(c_ref, s_abs, bf16_out)
    bad = np.nonzero(~(err <= tol))
    if bad[0].size:
        i = tuple(b[0] for b in bad)
        raise AssertionError("GEMM mismatch at %s: gpu %r ref %r S %r (%d bad)"
                             % (i, c_gpu[i], c_ref[i], s_abs[i], bad[0].size))
    zero = s_abs == 0
    assert np.all(c_gpu[zero] == 0)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where(s_abs > 0, np.abs(c_gpu.astype(np.float64) - c_ref) / s_abs, 0.0)
    return float(r.max()) if r.size else 0.0


def bf16_out_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(bits)
