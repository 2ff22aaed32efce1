"""CPU oracle for the MX quantize / block-Hadamard / MX-GEMM path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
cpu_baseline leg use it; the product library never does, and nothing here
is shared with it.

Quantization and the rotation are plain C (`mx_oracle.c`, loaded with
ctypes).  The GEMM is the definition of the MX dot product written out with
a library primitive: both operands are dequantized exactly to float64
(code * 2^(S-127)) and multiplied with numpy's float64 matmul; the
tolerance reference S_abs = sum_k |a_mk * b_nk| is the same product on
absolute values.  MX products of E4M3/E5M2/E2M1 codes with E8M0 scales are
exact in float64, so the only rounding is float64 summation (relative error
~K * 2^-53, far below the fp32 tolerance the GPU result is held to).

Formats follow the Lumen page (section 1: E4M3, E5M2) and the FP4-training
article (sections 02, 04: MXFP4 = E2M1 with per-block scales); block size 32
from the MindSpeed-LLM FSDP2 page (recipe dynamic_MX-1-1-32).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC_PATH = os.path.join(HERE, "mx_oracle.c")

FMT_CODES = {"e4m3": 0, "e5m2": 1, "e2m1": 2}
MAXNORM = {"e4m3": 448.0, "e5m2": 57344.0, "e2m1": 6.0}
EMAX = {"e4m3": 8, "e5m2": 15, "e2m1": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP, no fast-math)."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-Wall", "-Wextra", SRC_PATH, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
        L.oracle_hadamard_c.restype = ctypes.c_float
        L.oracle_hadamard32_f32.argtypes = [P, u32, P]
        L.oracle_hadamard32_f32.restype = None
        L.oracle_philox4x32_10.argtypes = [P, P, P]
        L.oracle_philox4x32_10.restype = None
        for name, args in {
            "oracle_e8m0_many": [P, i64, i32, P],
            "oracle_cast_many": [P, P, i64, i32, P],
            "oracle_decode_many": [P, i64, i32, P],
            "oracle_quantize_rows": [P, i64, i64, i64, i32, P, P],
            "oracle_quantize_rows_f64": [P, i64, i64, i32, P, P],
            "oracle_quantize_transpose": [P, i64, i64, i64, i32, P, P],
            "oracle_hadamard32_quantize": [P, i64, i64, i64, u32, i32, P, P],
            "oracle_dequantize": [P, P, i64, i64, i32, P],
            "oracle_cast_sr_many": [P, P, P, i64, i32, P],
            "oracle_sr_words": [ctypes.c_uint64, i64, i64, P],
            "oracle_quantize_transpose_sr": [P, i64, i64, i64, i32, u32, ctypes.c_uint64, i32, P, P],
        }.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(rc: int) -> None:
    if rc != 0:
        raise ValueError("oracle rejected its arguments")


def code_cols(n: int, fmt: str) -> int:
    """bytes per row holding n elements"""
    return n // 2 if fmt == "e2m1" else n


# --------------------------------------------------------------------------
# element-level entry points (used by the pins)

def hadamard_c() -> float:
    return float(lib().oracle_hadamard_c())


def hadamard32_f32(x: np.ndarray, mask: int = 0) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(32)
    y = np.empty(32, dtype=np.float32)
    lib().oracle_hadamard32_f32(_ptr(x), mask & 0xFFFFFFFF, _ptr(y))
    return y


def e8m0(amax: np.ndarray, fmt: str) -> np.ndarray:
    a = np.ascontiguousarray(amax, dtype=np.float64).ravel()
    out = np.empty(a.size, dtype=np.uint8)
    _check(lib().oracle_e8m0_many(_ptr(a), a.size, FMT_CODES[fmt], _ptr(out)))
    return out.reshape(np.shape(amax))


def cast(v: np.ndarray, e: np.ndarray, fmt: str) -> np.ndarray:
    """element codes (one per byte, unpacked) of v * 2^-e"""
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    e = np.ascontiguousarray(np.broadcast_to(e, v.shape), dtype=np.int32).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    _check(lib().oracle_cast_many(_ptr(v), _ptr(e), v.size, FMT_CODES[fmt], _ptr(out)))
    return out


def philox4x32_10(ctr, key) -> np.ndarray:
    """one Philox4x32-10 block: four 32-bit counter words, two key words -> four words"""
    c = np.ascontiguousarray(ctr, dtype=np.uint32).reshape(4)
    k = np.ascontiguousarray(key, dtype=np.uint32).reshape(2)
    out = np.empty(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_words(seed: int, n: int, start: int = 0) -> np.ndarray:
    """the random words of output elements start .. start+n-1 under `seed`"""
    out = np.empty(n, dtype=np.uint32)
    _check(lib().oracle_sr_words(seed & (2**64 - 1), start, n, _ptr(out)))
    return out


def cast_sr(v: np.ndarray, e: np.ndarray, r: np.ndarray, fmt: str) -> np.ndarray:
    """stochastically rounded element codes of v * 2^-e with random words r"""
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    e = np.ascontiguousarray(np.broadcast_to(e, v.shape), dtype=np.int32).ravel()
    r = np.ascontiguousarray(np.broadcast_to(r, v.shape), dtype=np.uint32).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    _check(lib().oracle_cast_sr_many(_ptr(v), _ptr(e), _ptr(r), v.size, FMT_CODES[fmt], _ptr(out)))
    return out


def decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    out = np.empty(c.size, dtype=np.float64)
    _check(lib().oracle_decode_many(_ptr(c), c.size, FMT_CODES[fmt], _ptr(out)))
    return out.reshape(np.shape(codes))


# --------------------------------------------------------------------------
# tensor-level entry points, one per library call

def quantize(x_bits: np.ndarray, fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """row mode: bf16 bits [rows x cols] -> (codes, scales)"""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.empty((rows, code_cols(cols, fmt)), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    _check(lib().oracle_quantize_rows(_ptr(x), rows, cols, cols, FMT_CODES[fmt], _ptr(codes), _ptr(scales)))
    return codes, scales


def quantize_f64(x: np.ndarray, fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """row mode on exact float64 values"""
    x = np.ascontiguousarray(x, dtype=np.float64)
    rows, cols = x.shape
    codes = np.empty((rows, code_cols(cols, fmt)), dtype=np.uint8)
    scales = np.empty((rows, cols // 32), dtype=np.uint8)
    _check(lib().oracle_quantize_rows_f64(_ptr(x), rows, cols, FMT_CODES[fmt], _ptr(codes), _ptr(scales)))
    return codes, scales


def quantize_transpose(x_bits: np.ndarray, fmt: str) -> Tuple[np.ndarray, np.ndarray]:
    """transposed mode: bf16 bits [rows x cols] -> codes [cols x rows(/2)], scales [cols x rows/32]"""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.empty((cols, code_cols(rows, fmt)), dtype=np.uint8)
    scales = np.empty((cols, rows // 32), dtype=np.uint8)
    _check(lib().oracle_quantize_transpose(_ptr(x), rows, cols, cols, FMT_CODES[fmt], _ptr(codes), _ptr(scales)))
    return codes, scales


def hadamard32_quantize(x_bits: np.ndarray, fmt: str, sign_mask: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """rotation of each 32-row block, then transposed-mode quantization"""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.empty((cols, code_cols(rows, fmt)), dtype=np.uint8)
    scales = np.empty((cols, rows // 32), dtype=np.uint8)
    _check(lib().oracle_hadamard32_quantize(_ptr(x), rows, cols, cols, sign_mask & 0xFFFFFFFF,
                                            FMT_CODES[fmt], _ptr(codes), _ptr(scales)))
    return codes, scales


def quantize_transpose_sr(x_bits: np.ndarray, fmt: str, seed: int, rotate: bool = False,
                          sign_mask: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """transposed mode (after the rotation if `rotate`) with stochastic rounding"""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.empty((cols, code_cols(rows, fmt)), dtype=np.uint8)
    scales = np.empty((cols, rows // 32), dtype=np.uint8)
    _check(lib().oracle_quantize_transpose_sr(_ptr(x), rows, cols, cols, int(bool(rotate)), sign_mask & 0xFFFFFFFF,
                                              seed & (2**64 - 1), FMT_CODES[fmt], _ptr(codes), _ptr(scales)))
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """exact float64 values [rows x K] of an MX operand"""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, nb = scales.shape
    K = nb * 32
    out = np.empty((rows, K), dtype=np.float64)
    _check(lib().oracle_dequantize(_ptr(codes), _ptr(scales), rows, K, FMT_CODES[fmt], _ptr(out)))
    return out


def gemm(a_codes: np.ndarray, a_scales: np.ndarray, fa: str,
         b_codes: np.ndarray, b_scales: np.ndarray, fb: str,
         rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """C[m, n] = sum_k A[m, k] * B[n, k] on MX operands, float64; also S_abs.

    `rows` restricts the result to those rows of A (sampled checks at full size).
    """
    if rows is not None:
        idx = np.asarray(rows, dtype=np.int64)
        a_codes, a_scales = a_codes[idx], a_scales[idx]
    A = dequantize(a_codes, a_scales, fa)
    B = dequantize(b_codes, b_scales, fb)
    if A.shape[1] != B.shape[1]:
        raise ValueError("K mismatch")
    C = A @ B.T
    S = np.abs(A) @ np.abs(B).T
    return C, S
