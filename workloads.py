"""Seeded synthetic inputs for the MX quantize / block-Hadamard / MX-GEMM path.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It holds no arithmetic of the method itself: it draws random
numbers, scales them, plants outliers and zero blocks, and rounds the result
to bf16 (round-to-nearest-even, torch's float32->bfloat16 cast).  Everything
downstream (block amax, E8M0 scales, element casts, rotation, GEMM) lives in
`oracle/` (reference) or in the HIP library (product), never here.

The workloads stand in for the Llama-3.1 pre-training runs that the FP4
training write-up (hzrcw.cc article, section 03) and the Lumen page (section
"LLaMA 3.1 预训练") describe: same linear-layer shapes, synthetic values.

Recipe (applies to every tensor):
  * generator: numpy PCG64 seeded with SeedSequence([seed, config, tensor, chunk]);
    a tensor is drawn in fixed chunks of CHUNK_ROWS rows so the bytes do not
    depend on the number of threads;
  * "normal(sigma)": standard normal float32 draws times sigma;
  * "t3(scale)": Student-t with 3 degrees of freedom (float64 draws) times scale;
  * outlier channels: round(frac * cols) column indices chosen without
    replacement (by a generator seeded with [seed, config, tensor, 1<<20]) are
    multiplied by the factor;
  * outlier entries: a Bernoulli(p) mask per entry, multiplied by the factor;
  * zero blocks: listed (row0, row1, col0, col1) rectangles are set to 0;
  * final float32 -> bf16 by round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

CHUNK_ROWS = 256
DEFAULT_SEED = 0

# format names, as in the OCP MX element types
E4M3, E5M2, E2M1 = "e4m3", "e5m2", "e2m1"


@dataclasses.dataclass(frozen=True)
class TensorSpec:
    name: str
    rows: int
    cols: int
    dist: str                      # "normal" or "t3"
    scale: float = 1.0
    outlier_channels: float = 0.0  # fraction of columns scaled
    outlier_entries: float = 0.0   # Bernoulli probability per entry
    outlier_factor: float = 1.0
    zero_blocks: Tuple[Tuple[int, int, int, int], ...] = ()


@dataclasses.dataclass(frozen=True)
class QuantSpec:
    """One quantize call: `kind` is "row", "transpose" or "hadamard"."""
    name: str        # name of the produced MX operand
    tensor: str      # source tensor
    kind: str
    fmt: str
    sign_mask: int = 0


@dataclasses.dataclass(frozen=True)
class GemmSpec:
    """C[M x N] = A[M x K] . B[N x K]^T on two MX operands."""
    name: str
    a: str
    b: str
    M: int
    N: int
    K: int
    out: str         # "f32" or "bf16"


@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    name: str
    tensors: Tuple[TensorSpec, ...]
    quants: Tuple[QuantSpec, ...]
    gemms: Tuple[GemmSpec, ...]

    def tensor(self, name: str) -> TensorSpec:
        for t in self.tensors:
            if t.name == name:
                return t
        raise KeyError(name)

    def quant(self, name: str) -> QuantSpec:
        for q in self.quants:
            if q.name == name:
                return q
        raise KeyError(name)


def _act(name, rows, cols):
    return TensorSpec(name, rows, cols, "normal", 1.0, outlier_channels=0.001,
                      outlier_factor=50.0)


def _weight(name, rows, cols, sigma):
    return TensorSpec(name, rows, cols, "normal", sigma)


def _grad(name, rows, cols):
    return TensorSpec(name, rows, cols, "t3", 1e-3)


T = 8192  # tokens per step in every Llama-3.1 configuration

CONFIGS: Tuple[Config, ...] = (
    # small MXFP8 correctness case: A through the row quantizer, B (stored K x N)
    # through the transposing quantizer, fp32 output
    Config(
        0, "mxfp8_e4m3_256x256x512",
        (
            TensorSpec("A", 256, 512, "normal", 1.0, outlier_entries=0.01,
                       outlier_factor=30.0, zero_blocks=((7, 8, 96, 128),)),
            TensorSpec("B", 512, 256, "normal", 1.0, outlier_entries=0.01,
                       outlier_factor=30.0, zero_blocks=((288, 320, 200, 201),)),
        ),
        (QuantSpec("qA", "A", "row", E4M3), QuantSpec("qB", "B", "transpose", E4M3)),
        (GemmSpec("AB", "qA", "qB", 256, 256, 512, "f32"),),
    ),
    # Llama-3.1-8B QKV projection, forward, MXFP8 E4M3
    Config(
        1, "llama31_8b_qkv_fprop_mxfp8",
        (_act("X", T, 4096), _weight("W", 6144, 4096, 0.02)),
        (QuantSpec("qX", "X", "row", E4M3), QuantSpec("qW", "W", "row", E4M3)),
        (GemmSpec("Y", "qX", "qW", T, 6144, 4096, "bf16"),),
    ),
    # Llama-3.1-8B gate+up projection, forward, MXFP4 E2M1
    Config(
        2, "llama31_8b_gateup_fprop_mxfp4",
        (_act("X", T, 4096), _weight("W", 28672, 4096, 0.02)),
        (QuantSpec("qX", "X", "row", E2M1), QuantSpec("qW", "W", "row", E2M1)),
        (GemmSpec("Y", "qX", "qW", T, 28672, 4096, "bf16"),),
    ),
    # Llama-3.1-8B weight gradient dW[14336 x 4096] = dY^T X over K = 8192 tokens,
    # both operands block-Hadamard rotated along tokens, MXFP4 E2M1
    Config(
        3, "llama31_8b_wgrad_mxfp4_hadamard",
        (_grad("dY", T, 14336), TensorSpec("X", T, 4096, "normal", 1.0)),
        (QuantSpec("qdY", "dY", "hadamard", E2M1), QuantSpec("qX", "X", "hadamard", E2M1)),
        (GemmSpec("dW", "qdY", "qX", 14336, 4096, T, "f32"),),
    ),
    # Llama-3.1-70B single-layer linear set (hidden 8192, MLP 28672, GQA 64/8 heads)
    Config(
        4, "llama31_70b_layer_linear_set",
        (
            _act("X_attn", T, 8192), _weight("W_qkv", 10240, 8192, 0.01), _grad("dY_qkv", T, 10240),
            _act("attn_out", T, 8192), _weight("W_o", 8192, 8192, 0.01), _grad("dY_o", T, 8192),
            _act("X_mlp", T, 8192), _weight("W_gu", 57344, 8192, 0.01), _grad("dY_gu", T, 57344),
            _act("h", T, 28672), _weight("W_down", 8192, 28672, 0.01), _grad("dY_down", T, 8192),
        ),
        (
            QuantSpec("qX_attn", "X_attn", "row", E4M3), QuantSpec("qW_qkv", "W_qkv", "row", E4M3),
            QuantSpec("qW_qkv_T", "W_qkv", "transpose", E4M3), QuantSpec("qdY_qkv", "dY_qkv", "row", E5M2),
            QuantSpec("qattn_out", "attn_out", "row", E4M3), QuantSpec("qW_o", "W_o", "row", E4M3),
            QuantSpec("qW_o_T", "W_o", "transpose", E4M3), QuantSpec("qdY_o", "dY_o", "row", E5M2),
            QuantSpec("qX_mlp", "X_mlp", "row", E4M3), QuantSpec("qW_gu", "W_gu", "row", E4M3),
            QuantSpec("qW_gu_T", "W_gu", "transpose", E4M3), QuantSpec("qdY_gu", "dY_gu", "row", E5M2),
            QuantSpec("qh", "h", "row", E4M3), QuantSpec("qW_down", "W_down", "row", E4M3),
            QuantSpec("qW_down_T", "W_down", "transpose", E4M3), QuantSpec("qdY_down", "dY_down", "row", E5M2),
            QuantSpec("qdY_down_H", "dY_down", "hadamard", E2M1), QuantSpec("qh_H", "h", "hadamard", E2M1),
        ),
        (
            GemmSpec("qkv_fprop", "qX_attn", "qW_qkv", T, 10240, 8192, "bf16"),
            GemmSpec("o_fprop", "qattn_out", "qW_o", T, 8192, 8192, "bf16"),
            GemmSpec("gu_fprop", "qX_mlp", "qW_gu", T, 57344, 8192, "bf16"),
            GemmSpec("down_fprop", "qh", "qW_down", T, 8192, 28672, "bf16"),
            GemmSpec("qkv_dgrad", "qdY_qkv", "qW_qkv_T", T, 8192, 10240, "bf16"),
            GemmSpec("o_dgrad", "qdY_o", "qW_o_T", T, 8192, 8192, "bf16"),
            GemmSpec("gu_dgrad", "qdY_gu", "qW_gu_T", T, 8192, 57344, "bf16"),
            GemmSpec("down_dgrad", "qdY_down", "qW_down_T", T, 28672, 8192, "bf16"),
            GemmSpec("down_wgrad", "qdY_down_H", "qh_H", 8192, 28672, T, "f32"),
        ),
    ),
    # One whole Llama-3.1-8B gate+up linear layer in the MXFP4 recipe (FP4-training
    # article, section 02: forward, activation-gradient and weight-gradient GEMMs in
    # MXFP4, the weight gradient's operands rotated): each source tensor is needed in
    # two forms, which the dual-direction quantizer produces from one read --
    # X: row (Fprop) + rotated (Wgrad); W: row (Fprop) + transposed (Dgrad);
    # dY: row (Dgrad) + rotated (Wgrad).
    Config(
        5, "llama31_8b_gateup_layer_mxfp4",
        (_act("X", T, 4096), _weight("W", 28672, 4096, 0.02), _grad("dY", T, 28672)),
        (
            QuantSpec("qX", "X", "row", E2M1), QuantSpec("qX_H", "X", "hadamard", E2M1),
            QuantSpec("qW", "W", "row", E2M1), QuantSpec("qW_T", "W", "transpose", E2M1),
            QuantSpec("qdY", "dY", "row", E2M1), QuantSpec("qdY_H", "dY", "hadamard", E2M1),
        ),
        (
            GemmSpec("fprop", "qX", "qW", T, 28672, 4096, "bf16"),
            GemmSpec("dgrad", "qdY", "qW_T", T, 4096, 28672, "bf16"),
            GemmSpec("wgrad", "qdY_H", "qX_H", 28672, 4096, T, "f32"),
        ),
    ),
)

# the dual-direction quantizations of that layer: (source, row-form operand, transposed-form operand)
LAYER_DUALS = (("X", "qX", "qX_H"), ("W", "qW", "qW_T"), ("dY", "qdY", "qdY_H"))


def config(index_or_name) -> Config:
    for c in CONFIGS:
        if c.index == index_or_name or c.name == index_or_name:
            return c
    raise KeyError(index_or_name)


def _tensor_index(cfg: Config, name: str) -> int:
    for i, t in enumerate(cfg.tensors):
        if t.name == name:
            return i
    raise KeyError(name)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def draw(spec: TensorSpec, config_index: int, tensor_index: int,
         seed: int = DEFAULT_SEED, rows: Optional[Tuple[int, int]] = None) -> np.ndarray:
    """Return the tensor as bf16 bit patterns, uint16 [rows x cols].

    `rows=(r0, r1)` draws only that row range (r0, r1 multiples of CHUNK_ROWS,
    or r1 == spec.rows); the bytes equal the same rows of the full tensor.
    """
    r0, r1 = (0, spec.rows) if rows is None else rows
    if r0 % CHUNK_ROWS or (r1 % CHUNK_ROWS and r1 != spec.rows) or not 0 <= r0 <= r1 <= spec.rows:
        raise ValueError("row range must be chunk aligned")
    cols = spec.cols
    out = np.empty((r1 - r0, cols), dtype=np.uint16)

    chan = None
    if spec.outlier_channels > 0:
        n_out = int(round(spec.outlier_channels * cols))
        g = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([seed, config_index, tensor_index, 1 << 20])))
        chan = np.sort(g.choice(cols, size=n_out, replace=False))

    def one_chunk(c0: int) -> None:
        c1 = min(c0 + CHUNK_ROWS, spec.rows)
        g = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([seed, config_index, tensor_index, c0 // CHUNK_ROWS])))
        n = (c1 - c0) * cols
        if spec.dist == "normal":
            v = g.standard_normal(n, dtype=np.float32)
            if spec.scale != 1.0:
                v *= np.float32(spec.scale)
        elif spec.dist == "t3":
            v = (g.standard_t(3, n) * spec.scale).astype(np.float32)
        else:
            raise ValueError(spec.dist)
        v = v.reshape(c1 - c0, cols)
        if spec.outlier_entries > 0:
            mask = g.random((c1 - c0, cols)) < spec.outlier_entries
            v[mask] *= np.float32(spec.outlier_factor)
        if chan is not None:
            v[:, chan] *= np.float32(spec.outlier_factor)
        for (zr0, zr1, zc0, zc1) in spec.zero_blocks:
            a, b = max(zr0, c0), min(zr1, c1)
            if a < b:
                v[a - c0:b - c0, zc0:zc1] = 0.0
        out[c0 - r0:c1 - r0] = _f32_to_bf16_bits(v)

    starts = list(range(r0, r1, CHUNK_ROWS))
    if len(starts) <= 1:
        for s in starts:
            one_chunk(s)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one_chunk, starts))
    return out


def draw_tensor(cfg: Config, name: str, seed: int = DEFAULT_SEED,
                rows: Optional[Tuple[int, int]] = None) -> np.ndarray:
    return draw(cfg.tensor(name), cfg.index, _tensor_index(cfg, name), seed, rows)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact; a bit shift)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)
