"""precision_block_amax_amd -- Python binding of libmx (include/mx.h) for AMD MI355X.

OCP-MX micro-scaling quantization (block 32, E8M0 scales, E4M3 / E5M2 / E2M1
elements), the fixed-sign 32-point block-Hadamard rotation used on the
weight-gradient path, and the MX-scaled GEMM, as hand-written gfx950 HIP
kernels behind a C ABI.

This module only marshals arguments: it checks tensor shapes, dtypes and
devices, allocates outputs with torch (device memory and streams are all
torch is used for), and calls the library on the current HIP stream.  Every
step of the computation runs in libmx.so; if the library is missing, loading
fails loudly.  Build it with ``python -m precision_block_amax_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple, Union

import torch

__all__ = [
    "E4M3", "E5M2", "E2M1", "MXError", "lib", "library_path", "code_cols",
    "quantize", "quantize_transpose", "hadamard32_quantize", "quantize_dual",
    "quantize_transpose_sr", "quantize_pair", "gemm", "fsdp_payload", "payload_views",
    "payload_width",
]

E4M3, E5M2, E2M1 = 0, 1, 2
_FORMATS = {"e4m3": E4M3, "e5m2": E5M2, "e2m1": E2M1, E4M3: E4M3, E5M2: E5M2, E2M1: E2M1}
OUT_F32, OUT_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmx.so")
_lib = None


class MXError(RuntimeError):
    """a libmx call returned a status other than MX_OK"""


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """the loaded libmx.so (raises if it has not been built)"""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise MXError("libmx.so not found at %s; build it with "
                          "`python -m precision_block_amax_amd.build`" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        P, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
        L.mx_quantize.argtypes = [P, i64, i64, i64, i32, P, P, P]
        L.mx_quantize_transpose.argtypes = [P, i64, i64, i64, i32, P, P, P]
        L.mx_hadamard32_quantize.argtypes = [P, i64, i64, i64, u32, i32, P, P, P]
        L.mx_quantize_dual.argtypes = [P, i64, i64, i64, i32, P, P, i32, i32, u32, P, P, P]
        L.mx_quantize_transpose_sr.argtypes = [P, i64, i64, i64, i32, u32, ctypes.c_uint64, i32, P, P, P]
        L.mx_quantize_pair.argtypes = [i32, i32, u32, P, i64, i64, i64, P, P, P, i64, i64, i64, P, P, P]
        L.mx_gemm.argtypes = [P, P, i32, P, P, i32, i64, i64, i64, P, i32, i64, P]
        L.mx_quantize_strided.argtypes = [P, i64, i64, i64, i32, P, i64, P, i64, P]
        L.mx_gemm_strided.argtypes = [P, i64, P, i64, i32, P, i64, P, i64, i32, i64, i64, i64, P, i32, i64, P]
        L.mx_quantize_transpose_panels.argtypes = [P, i64, i64, i64, i32, P, P, P]
        L.mx_hadamard32_quantize_panels.argtypes = [P, i64, i64, i64, u32, i32, P, P, P]
        L.mx_gemm_layout.argtypes = [P, i32, P, i32, P, i32, P, i32, i64, i64, i64, P, i32, i64, P]
        L.mx_quantize_dual_panels.argtypes = [P, i64, i64, i64, i32, P, P, i32, i32, u32, P, P, P]
        for fn in (L.mx_quantize, L.mx_quantize_transpose, L.mx_hadamard32_quantize, L.mx_quantize_dual,
                   L.mx_quantize_transpose_sr, L.mx_quantize_pair, L.mx_gemm, L.mx_quantize_strided,
                   L.mx_gemm_strided, L.mx_quantize_transpose_panels, L.mx_hadamard32_quantize_panels,
                   L.mx_gemm_layout, L.mx_quantize_dual_panels):
            fn.restype = ctypes.c_int
        L.mx_status_string.argtypes = [ctypes.c_int]
        L.mx_status_string.restype = ctypes.c_char_p
        L.mx_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _fmt(f: Union[str, int]) -> int:
    try:
        return _FORMATS[f.lower() if isinstance(f, str) else f]
    except KeyError:
        raise ValueError("unknown MX format %r" % (f,)) from None


def code_cols(n: int, fmt: Union[str, int]) -> int:
    """bytes holding n elements of a row"""
    return n // 2 if _fmt(fmt) == E2M1 else n


def _check(status: int) -> None:
    if status != 0:
        raise MXError(lib().mx_status_string(status).decode())


def _stream(device: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _check_bf16_2d(x: torch.Tensor) -> None:
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("expected a 2-D bf16 tensor on a GPU")
    if x.stride(1) != 1 and x.numel() > 0:
        raise ValueError("the last dimension must be contiguous")


def _outputs(device, rows_out: int, k: int, fmt: int, out, panels: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    shape_c, shape_s = (rows_out, code_cols(k, fmt)), (rows_out, k // 32)
    if panels:  # K-panel layout: [K panels x rows x 128 bytes]
        shape_c = (code_cols(k, fmt) // 128, rows_out, 128)
    if out is None:
        return (torch.empty(shape_c, dtype=torch.uint8, device=device),
                torch.empty(shape_s, dtype=torch.uint8, device=device))
    codes, scales = out
    for t, shp in ((codes, shape_c), (scales, shape_s)):
        if t.dtype != torch.uint8 or tuple(t.shape) != shp or not t.is_contiguous() or t.device != device:
            raise ValueError("output buffer must be contiguous uint8 of shape %s" % (shp,))
    return codes, scales


def _ldx(x: torch.Tensor) -> int:
    return x.stride(0) if x.shape[0] > 1 else x.shape[1]


def _row_strided(t: torch.Tensor, shape, device) -> int:
    """row stride in bytes of a uint8 [rows x width] view with contiguous rows"""
    if t.dtype != torch.uint8 or tuple(t.shape) != tuple(shape) or t.device != device:
        raise ValueError("expected a uint8 tensor of shape %s on %s" % (tuple(shape), device))
    if t.numel() and t.stride(1) != 1:
        raise ValueError("rows must be contiguous")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def quantize(x: torch.Tensor, fmt, out=None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mx_quantize: blocks of 32 along the last dim; codes [R x C(/2)], scales [R x C/32].
    `out` = (codes, scales) may be row-strided views (e.g. of an FSDP2 payload,
    see fsdp_payload); those go through mx_quantize_strided."""
    _check_bf16_2d(x)
    f = _fmt(fmt)
    rows, cols = x.shape
    if out is not None and not (out[0].is_contiguous() and out[1].is_contiguous()):
        codes, scales = out
        ldc = _row_strided(codes, (rows, code_cols(cols, f)), x.device)
        lds = _row_strided(scales, (rows, cols // 32), x.device)
        _check(lib().mx_quantize_strided(_ptr(x), rows, cols, _ldx(x), f, _ptr(codes), ldc, _ptr(scales), lds,
                                         _stream(x.device, stream)))
        return codes, scales
    codes, scales = _outputs(x.device, rows, cols, f, out)
    _check(lib().mx_quantize(_ptr(x), rows, cols, _ldx(x), f, _ptr(codes), _ptr(scales),
                             _stream(x.device, stream)))
    return codes, scales


def payload_width(K: int, fmt) -> int:
    """bytes per row of an FSDP2 payload: the row's codes, its K/32 scales, padded to 16"""
    return (code_cols(K, _fmt(fmt)) + K // 32 + 15) // 16 * 16


def payload_views(payload: torch.Tensor, K: int, fmt) -> Tuple[torch.Tensor, torch.Tensor]:
    """(codes, scales) views of an FSDP2 payload [rows x payload_width(K)]: each row holds a
    weight row's codes followed by its scales (mx_quantize_strided)"""
    cb = code_cols(K, _fmt(fmt))
    if payload.dim() != 2 or payload.shape[1] != payload_width(K, fmt) or payload.dtype != torch.uint8:
        raise ValueError("payload must be uint8 [rows x %d]" % payload_width(K, fmt))
    return payload[:, :cb], payload[:, cb:cb + K // 32]


def fsdp_payload(w_rows: torch.Tensor, fmt, out: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """One rank's FSDP2 all-gather payload: its slab of weight rows [rows x K] (dim-0 shard)
    quantized into one buffer of rows [codes | scales].  The ranks' payloads concatenated in
    rank order are the whole weight's payload; payload_views() of it is an mx_gemm operand."""
    _check_bf16_2d(w_rows)
    f = _fmt(fmt)
    rows, K = w_rows.shape
    width = payload_width(K, f)
    if out is None:
        out = torch.empty((rows, width), dtype=torch.uint8, device=w_rows.device)
    elif out.dtype != torch.uint8 or tuple(out.shape) != (rows, width) or not out.is_contiguous():
        raise ValueError("payload buffer must be contiguous uint8 [%d x %d]" % (rows, width))
    codes, scales = payload_views(out, K, f)
    ldp = width
    _check(lib().mx_quantize_strided(_ptr(w_rows), rows, K, _ldx(w_rows), f, _ptr(codes), ldp, _ptr(scales), ldp,
                                     _stream(w_rows.device, stream)))
    return out


_LAYOUTS = ("rows", "panels")


def _panels(layout: str) -> bool:
    if layout not in _LAYOUTS:
        raise ValueError("layout must be one of %s" % (_LAYOUTS,))
    return layout == "panels"


def quantize_transpose(x: torch.Tensor, fmt, out=None, stream=None, layout: str = "rows") -> Tuple[torch.Tensor, torch.Tensor]:
    """mx_quantize_transpose: blocks of 32 along dim 0; codes [C x R(/2)], scales [C x R/32].
    layout="panels": mx_quantize_transpose_panels, codes [R(/2) / 128 x C x 128] (K-panel layout)"""
    _check_bf16_2d(x)
    f = _fmt(fmt)
    rows, cols = x.shape
    pan = _panels(layout)
    codes, scales = _outputs(x.device, cols, rows, f, out, pan)
    fn = lib().mx_quantize_transpose_panels if pan else lib().mx_quantize_transpose
    _check(fn(_ptr(x), rows, cols, _ldx(x), f, _ptr(codes), _ptr(scales), _stream(x.device, stream)))
    return codes, scales


def quantize_dual(x: torch.Tensor, fmt_row, fmt_t, rotate: bool = False, sign_mask: int = 0, out=None,
                  stream=None, layout: str = "rows") -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """mx_quantize_dual: (codes_row, scales_row, codes_t, scales_t) from one read of x; the row
    form as quantize(x, fmt_row), the transposed form as quantize_transpose(x, fmt_t) or, with
    rotate, hadamard32_quantize(x, fmt_t, sign_mask).  `out` is a 4-tuple of output tensors.
    layout="panels": mx_quantize_dual_panels, both forms' codes in the K-panel layout."""
    _check_bf16_2d(x)
    fr, ft = _fmt(fmt_row), _fmt(fmt_t)
    rows, cols = x.shape
    pan = _panels(layout)
    cr, sr = _outputs(x.device, rows, cols, fr, None if out is None else out[:2], pan)
    ct, st = _outputs(x.device, cols, rows, ft, None if out is None else out[2:], pan)
    fn = lib().mx_quantize_dual_panels if pan else lib().mx_quantize_dual
    _check(fn(_ptr(x), rows, cols, _ldx(x), fr, _ptr(cr), _ptr(sr), ft, 1 if rotate else 0, sign_mask & 0xFFFFFFFF,
              _ptr(ct), _ptr(st), _stream(x.device, stream)))
    return cr, sr, ct, st


def hadamard32_quantize(x: torch.Tensor, fmt, sign_mask: int = 0, out=None,
                        stream=None, layout: str = "rows") -> Tuple[torch.Tensor, torch.Tensor]:
    """mx_hadamard32_quantize: rotate each 32-row block, then transposed-mode quantize
    (layout="panels": mx_hadamard32_quantize_panels, codes in the K-panel layout)"""
    _check_bf16_2d(x)
    f = _fmt(fmt)
    rows, cols = x.shape
    pan = _panels(layout)
    codes, scales = _outputs(x.device, cols, rows, f, out, pan)
    fn = lib().mx_hadamard32_quantize_panels if pan else lib().mx_hadamard32_quantize
    _check(fn(_ptr(x), rows, cols, _ldx(x), sign_mask & 0xFFFFFFFF, f, _ptr(codes), _ptr(scales),
              _stream(x.device, stream)))
    return codes, scales


def quantize_transpose_sr(x: torch.Tensor, fmt, seed: int, rotate: bool = False, sign_mask: int = 0, out=None,
                          stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mx_quantize_transpose_sr: quantize_transpose (or, with rotate, hadamard32_quantize) with
    stochastic rounding driven by the Philox4x32-10 stream of `seed`"""
    _check_bf16_2d(x)
    f = _fmt(fmt)
    rows, cols = x.shape
    codes, scales = _outputs(x.device, cols, rows, f, out)
    _check(lib().mx_quantize_transpose_sr(_ptr(x), rows, cols, _ldx(x), 1 if rotate else 0, sign_mask & 0xFFFFFFFF,
                                          seed & (2 ** 64 - 1), f, _ptr(codes), _ptr(scales),
                                          _stream(x.device, stream)))
    return codes, scales


_PAIR_MODES = {"row": 0, "transpose": 1, "hadamard": 2, "transpose_panels": 3, "hadamard_panels": 4}


def quantize_pair(mode: str, x0: torch.Tensor, x1: torch.Tensor, fmt, sign_mask: int = 0, out0=None, out1=None,
                  stream=None):
    """mx_quantize_pair: both operands of a GEMM in one launch, each exactly as quantize
    (mode "row"), quantize_transpose ("transpose") or hadamard32_quantize ("hadamard", with
    sign_mask) would quantize it; "transpose_panels" and "hadamard_panels" write the codes in
    the K-panel layout (layout="panels").  Returns ((codes0, scales0), (codes1, scales1))."""
    if mode not in _PAIR_MODES:
        raise ValueError("mode must be one of %s" % sorted(_PAIR_MODES))
    _check_bf16_2d(x0)
    _check_bf16_2d(x1)
    if x0.device != x1.device:
        raise ValueError("both tensors must be on the same device")
    f = _fmt(fmt)
    outs = []
    for x, out in ((x0, out0), (x1, out1)):
        rows, cols = x.shape
        outs.append(_outputs(x.device, rows, cols, f, out) if mode == "row" else
                    _outputs(x.device, cols, rows, f, out, mode.endswith("_panels")))
    (c0, s0), (c1, s1) = outs
    _check(lib().mx_quantize_pair(_PAIR_MODES[mode], f, sign_mask & 0xFFFFFFFF,
                                  _ptr(x0), x0.shape[0], x0.shape[1], _ldx(x0), _ptr(c0), _ptr(s0),
                                  _ptr(x1), x1.shape[0], x1.shape[1], _ldx(x1), _ptr(c1), _ptr(s1),
                                  _stream(x0.device, stream)))
    return (c0, s0), (c1, s1)


def gemm(a_codes: torch.Tensor, a_scales: torch.Tensor, fa, b_codes: torch.Tensor,
         b_scales: torch.Tensor, fb, out_dtype: torch.dtype = torch.bfloat16,
         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """mx_gemm: C[M x N] = A[M x K] . B[N x K]^T on MX operands.  Operands may be
    row-strided uint8 views (rows contiguous), e.g. payload_views() of a gathered
    FSDP2 payload; those go through mx_gemm_strided.  Codes in the K-panel layout
    (3-D, [K bytes / 128 x rows x 128], as quantize_transpose(layout="panels")
    writes them) go through mx_gemm_layout."""
    fa_, fb_ = _fmt(fa), _fmt(fb)
    M, kb = a_scales.shape
    N, kb2 = b_scales.shape
    K = 32 * kb
    if kb2 != kb:
        raise ValueError("A and B disagree on K")
    dev = a_codes.device
    if not a_codes.is_cuda:
        raise ValueError("operands must be on a GPU")
    panel = [t.dim() == 3 for t in (a_codes, b_codes)]
    if any(panel):
        for t, rows, f, pn in ((a_codes, M, fa_, panel[0]), (b_codes, N, fb_, panel[1])):
            shp = (code_cols(K, f) // 128, rows, 128) if pn else (rows, code_cols(K, f))
            if t.dtype != torch.uint8 or tuple(t.shape) != shp or t.device != dev or not t.is_contiguous():
                raise ValueError("expected a contiguous uint8 tensor of shape %s on %s" % (shp, dev))
        for t, shp in ((a_scales, (M, kb)), (b_scales, (N, kb))):
            if t.dtype != torch.uint8 or tuple(t.shape) != shp or t.device != dev or not t.is_contiguous():
                raise ValueError("expected a contiguous uint8 tensor of shape %s on %s" % (shp, dev))
    else:
        lds = [_row_strided(t, shp, dev) for t, shp in ((a_codes, (M, code_cols(K, fa_))), (a_scales, (M, kb)),
                                                         (b_codes, (N, code_cols(K, fb_))), (b_scales, (N, kb)))]
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    elif out.dtype != out_dtype or tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError("bad output buffer")
    ldc = out.stride(0) if M > 1 else N
    o = OUT_BF16 if out_dtype == torch.bfloat16 else OUT_F32
    if any(panel):
        _check(lib().mx_gemm_layout(_ptr(a_codes), int(panel[0]), _ptr(a_scales), fa_, _ptr(b_codes), int(panel[1]),
                                    _ptr(b_scales), fb_, M, N, K, _ptr(out), o, ldc, _stream(dev, stream)))
    elif all(t.is_contiguous() for t in (a_codes, a_scales, b_codes, b_scales)):
        _check(lib().mx_gemm(_ptr(a_codes), _ptr(a_scales), fa_, _ptr(b_codes), _ptr(b_scales), fb_,
                             M, N, K, _ptr(out), o, ldc, _stream(dev, stream)))
    else:
        _check(lib().mx_gemm_strided(_ptr(a_codes), lds[0], _ptr(a_scales), lds[1], fa_, _ptr(b_codes), lds[2],
                                     _ptr(b_scales), lds[3], fb_, M, N, K, _ptr(out), o, ldc, _stream(dev, stream)))
    return out
