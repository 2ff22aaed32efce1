"""GPU parity of mx_quantize_pair (both operands of one GEMM in one launch):
each tensor's codes and scales bit-exact to the oracle and to the single call
of its mode (mx_quantize, mx_quantize_transpose, mx_hadamard32_quantize), for
tensors of different shapes, ragged tails, a grid whose rows outrun the
shorter tensor, strided and unaligned tensors (which take two launches), an
empty tensor, one tensor passed twice, and the full-size operand pairs of the
Llama-3.1-8B layers as the benchmark quantizes them."""
import numpy as np
import pytest

import oracle
import workloads
from helpers import to_dev_bf16, to_host

pytestmark = pytest.mark.gpu
FMTS = ("e4m3", "e5m2", "e2m1")
MASK = 0x9E3779B9


@pytest.fixture(scope="module")
def mx():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_block_amax_amd as m
    m.lib()
    return m


def _bf16_bits(rng, rows, cols):
    """normal values with ~1% of entries x40, rounded to bf16 (nearest, ties to even)"""
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    v[rng.random((rows, cols)) < 0.01] *= 40.0
    u = v.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _oracle(mode, x, fmt, mask):
    if mode == "row":
        return oracle.quantize(x, fmt)
    if mode == "transpose":
        return oracle.quantize_transpose(x, fmt)
    return oracle.hadamard32_quantize(x, fmt, mask)


def _single(mx, mode, x, fmt, mask):
    if mode == "row":
        return mx.quantize(x, fmt)
    if mode == "transpose":
        return mx.quantize_transpose(x, fmt)
    return mx.hadamard32_quantize(x, fmt, mask)


def _eq(got, want, what):
    g = (to_host(got[0]), to_host(got[1]))
    w = (want[0] if isinstance(want[0], np.ndarray) else to_host(want[0]),
         want[1] if isinstance(want[1], np.ndarray) else to_host(want[1]))
    assert g[1].shape == w[1].shape and np.array_equal(g[1], w[1]), "%s: scales differ" % what
    assert g[0].shape == w[0].shape and np.array_equal(g[0], w[0]), "%s: codes differ" % what


# (rows, cols) of the two tensors: different shapes, ragged column tails, and (transposed
# modes) 17 row blocks against 3, so part of the grid lies below the second tensor
SHAPES = {"row": ((97, 224), (300, 4128)), "transpose": ((544, 300), (96, 260)), "hadamard": ((544, 300), (96, 260))}


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", ["row", "transpose", "hadamard"])
def test_pair_matches_oracle_and_single_calls(mx, mode, fmt):
    rng = np.random.default_rng(FMTS.index(fmt) * 3 + ["row", "transpose", "hadamard"].index(mode))
    (r0, c0), (r1, c1) = SHAPES[mode]
    x0, x1 = _bf16_bits(rng, r0, c0), _bf16_bits(rng, r1, c1)
    d0, d1 = to_dev_bf16(x0), to_dev_bf16(x1)
    print("case", mode, fmt, x0.shape, x1.shape, flush=True)
    p0, p1 = mx.quantize_pair(mode, d0, d1, fmt, MASK)
    _eq(p0, _oracle(mode, x0, fmt, MASK), "first tensor vs oracle")
    _eq(p1, _oracle(mode, x1, fmt, MASK), "second tensor vs oracle")
    _eq(p0, _single(mx, mode, d0, fmt, MASK), "first tensor vs single call")
    _eq(p1, _single(mx, mode, d1, fmt, MASK), "second tensor vs single call")


@pytest.mark.parametrize("mode", ["row", "transpose", "hadamard"])
def test_pair_two_launch_fallback(mx, mode):
    """a strided second tensor (row mode) or an unaligned first one (transposed modes)
    needs another kernel variant than its partner: two launches, same results"""
    import torch
    rng = np.random.default_rng(11)
    big0, big1 = _bf16_bits(rng, 128, 264), _bf16_bits(rng, 96, 200)
    t0, t1 = to_dev_bf16(big0), to_dev_bf16(big1)
    if mode == "row":
        v0, v1 = t0[:, :256], t1[:, :160]               # strided (ldx > cols)
        h0, h1 = big0[:, :256], big1[:, :160]
    else:
        v0, v1 = t0[:, 1:258], t1[:, :192]              # first one starts 2 bytes into its rows
        h0, h1 = big0[:, 1:258], big1[:, :192]
    assert v0.stride(1) == 1 and v1.stride(1) == 1
    print("case", mode, tuple(v0.shape), tuple(v1.shape), flush=True)
    p0, p1 = mx.quantize_pair(mode, v0, v1, "e2m1", MASK)
    _eq(p0, _oracle(mode, np.ascontiguousarray(h0), "e2m1", MASK), "first tensor")
    _eq(p1, _oracle(mode, np.ascontiguousarray(h1), "e2m1", MASK), "second tensor")


@pytest.mark.parametrize("mode", ["row", "hadamard"])
def test_pair_empty_tensor_and_same_tensor_twice(mx, mode):
    import torch
    rng = np.random.default_rng(5)
    x = _bf16_bits(rng, 64, 96)
    d = to_dev_bf16(x)
    empty = torch.empty((0, 96), dtype=torch.bfloat16, device="cuda")
    p0, p1 = mx.quantize_pair(mode, d, empty, "e4m3", MASK)
    _eq(p0, _oracle(mode, x, "e4m3", MASK), "non-empty tensor beside an empty one")
    assert p1[0].numel() == 0 and p1[1].numel() == 0
    q0, q1 = mx.quantize_pair(mode, d, d, "e4m3", MASK)  # the inputs may overlap: they are only read
    _eq(q0, p0, "same tensor, first output")
    _eq(q1, p0, "same tensor, second output")


# the benchmark step's operand pairs at full size: config, first, second, mode, format, mask
STEP_PAIRS = [(1, "X", "W", "row", "e4m3", 0), (2, "X", "W", "row", "e2m1", 0),
              (3, "dY", "X", "hadamard", "e2m1", 0)]


@pytest.mark.parametrize("ci,n0,n1,mode,fmt,mask", STEP_PAIRS)
def test_pair_full_size_step_operands(mx, ci, n0, n1, mode, fmt, mask):
    """as the benchmark launches them; each equals its single call, which the
    quantizer tests pin to the oracle on these same tensors"""
    cfg = workloads.config(ci)
    d0, d1 = to_dev_bf16(workloads.draw_tensor(cfg, n0)), to_dev_bf16(workloads.draw_tensor(cfg, n1))
    print("case", cfg.name, n0, n1, mode, fmt, tuple(d0.shape), tuple(d1.shape), flush=True)
    p0, p1 = mx.quantize_pair(mode, d0, d1, fmt, mask)
    _eq(p0, _single(mx, mode, d0, fmt, mask), "%s/%s" % (cfg.name, n0))
    _eq(p1, _single(mx, mode, d1, fmt, mask), "%s/%s" % (cfg.name, n1))
