"""The C-ABI library on the host: it loads, exports every function include/mx.h
declares, and rejects bad arguments before any HIP call (so these checks
need no GPU; pointer arguments are only compared, never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mx.h")

OK, INVALID, UNSUPPORTED, HIPERR = 0, 1, 2, 3
E4M3, E5M2, E2M1 = 0, 1, 2
P, i64, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32


@pytest.fixture(scope="module")
def L():
    from precision_block_amax_amd import build as libbuild
    if not os.path.exists(libbuild.LIB_PATH):
        libbuild.build()
    lib = ctypes.CDLL(libbuild.LIB_PATH)
    lib.mx_quantize.argtypes = [P, i64, i64, i64, i32, P, P, P]
    lib.mx_quantize_transpose.argtypes = [P, i64, i64, i64, i32, P, P, P]
    lib.mx_hadamard32_quantize.argtypes = [P, i64, i64, i64, u32, i32, P, P, P]
    lib.mx_quantize_dual.argtypes = [P, i64, i64, i64, i32, P, P, i32, i32, u32, P, P, P]
    lib.mx_quantize_transpose_sr.argtypes = [P, i64, i64, i64, i32, u32, ctypes.c_uint64, i32, P, P, P]
    lib.mx_quantize_pair.argtypes = [i32, i32, u32, P, i64, i64, i64, P, P, P, i64, i64, i64, P, P, P]
    lib.mx_gemm.argtypes = [P, P, i32, P, P, i32, i64, i64, i64, P, i32, i64, P]
    lib.mx_quantize_strided.argtypes = [P, i64, i64, i64, i32, P, i64, P, i64, P]
    lib.mx_gemm_strided.argtypes = [P, i64, P, i64, i32, P, i64, P, i64, i32, i64, i64, i64, P, i32, i64, P]
    lib.mx_quantize_transpose_panels.argtypes = [P, i64, i64, i64, i32, P, P, P]
    lib.mx_hadamard32_quantize_panels.argtypes = [P, i64, i64, i64, u32, i32, P, P, P]
    lib.mx_gemm_layout.argtypes = [P, i32, P, i32, P, i32, P, i32, i64, i64, i64, P, i32, i64, P]
    lib.mx_quantize_dual_panels.argtypes = [P, i64, i64, i64, i32, P, P, i32, i32, u32, P, P, P]
    lib.mx_status_string.argtypes = [ctypes.c_int]
    lib.mx_status_string.restype = ctypes.c_char_p
    return lib


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mx_status_t|const char \*|int)\s*\*?\s*(mx_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert {"mx_quantize", "mx_quantize_transpose", "mx_hadamard32_quantize", "mx_quantize_dual",
            "mx_quantize_transpose_sr", "mx_quantize_pair", "mx_gemm", "mx_quantize_strided",
            "mx_gemm_strided", "mx_quantize_transpose_panels", "mx_hadamard32_quantize_panels",
            "mx_gemm_layout", "mx_quantize_dual_panels", "mx_status_string", "mx_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), "libmx.so does not export %s" % n


def test_version_and_status_strings(L):
    assert L.mx_version() == 100
    for code, name in [(OK, b"MX_OK"), (INVALID, b"MX_ERR_INVALID_ARG"), (UNSUPPORTED, b"MX_ERR_UNSUPPORTED"),
                       (HIPERR, b"MX_ERR_HIP"), (99, b"MX_ERR_UNKNOWN")]:
        assert L.mx_status_string(code) == name


X, C, S, C2, S2 = (P(a) for a in (0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000))


@pytest.mark.parametrize("fn", ["mx_quantize", "mx_quantize_transpose"])
def test_quantize_rejects(L, fn):
    f = getattr(L, fn)
    blocked_rows = fn != "mx_quantize"
    good_r, good_c = (64, 3) if blocked_rows else (3, 64)
    assert f(X, -1, 64, 64, E4M3, C, S, None) == INVALID                       # negative size
    assert f(X, good_r, good_c, good_c, 7, C, S, None) == INVALID              # unknown format
    bad_r, bad_c = (33, 3) if blocked_rows else (3, 33)
    assert f(X, bad_r, bad_c, bad_c, E4M3, C, S, None) == INVALID              # blocked dim % 32
    assert f(X, good_r, good_c, good_c - 1, E4M3, C, S, None) == INVALID      # ldx < cols
    assert f(None, good_r, good_c, good_c, E4M3, C, S, None) == INVALID        # NULL input
    assert f(X, good_r, good_c, good_c, E4M3, None, S, None) == INVALID        # NULL codes
    assert f(X, good_r, good_c, good_c, E4M3, X, S, None) == INVALID           # codes overlap x
    assert f(X, good_r, good_c, good_c, E4M3, C, P(0x20000010), None) == INVALID  # scales overlap codes
    assert f(None, 0, good_c, good_c, E4M3, None, None, None) == OK            # empty call
    assert f(None, good_r, 0, max(good_c, 0), E4M3, None, None, None) == OK


def test_hadamard_rejects(L):
    f = L.mx_hadamard32_quantize
    assert f(X, 33, 4, 4, 0, E2M1, C, S, None) == INVALID
    assert f(X, 64, 4, 4, 0x9E3779B9, 5, C, S, None) == INVALID
    assert f(X, 64, 4, 3, 0, E2M1, C, S, None) == INVALID
    assert f(None, 0, 4, 4, 0, E2M1, None, None, None) == OK


def test_sr_rejects(L):
    f = L.mx_quantize_transpose_sr
    assert f(X, 64, 4, 4, 2, 0, 1, E2M1, C, S, None) == INVALID             # rotate is 0 or 1
    assert f(X, 33, 4, 4, 0, 0, 1, E2M1, C, S, None) == INVALID             # rows % 32
    assert f(X, 64, 4, 4, 1, 0, 1, 5, C, S, None) == INVALID                # format
    assert f(X, 64, 4, 3, 1, 0, 1, E2M1, C, S, None) == INVALID             # ldx < cols
    assert f(X, 64, 4, 4, 1, 0, 1, E2M1, X, S, None) == INVALID             # codes overlap x
    assert f(X, 64, 4, 4, 1, 0, 1, E2M1, None, S, None) == INVALID
    assert f(None, 0, 4, 4, 1, 0, 1, E2M1, None, None, None) == OK          # empty


def test_dual_rejects(L):
    f = L.mx_quantize_dual
    args = lambda **k: [k.get("x", X), k.get("rows", 64), k.get("cols", 64), k.get("ldx", 64), k.get("fr", E4M3),
                        k.get("cr", C), k.get("sr", S), k.get("ft", E2M1), k.get("rot", 1), 0, k.get("ct", C2),
                        k.get("st", S2), None]
    assert f(*args(rot=2)) == INVALID                    # rotate is 0 or 1
    assert f(*args(rows=48)) == INVALID                  # rows % 32 (transposed form)
    assert f(*args(cols=48, ldx=48)) == INVALID          # cols % 32 (row form)
    assert f(*args(ft=9)) == INVALID
    assert f(*args(ct=C)) == INVALID                     # the two code buffers overlap
    assert f(*args(st=P(0x30000040))) == INVALID         # scale buffers overlap
    assert f(*args(sr=P(0x40000000))) == INVALID         # row scales inside the transposed codes
    assert f(*args(ldx=63)) == INVALID
    assert f(*args(x=None)) == INVALID
    assert f(*args(rows=0, x=None, cr=None, sr=None, ct=None, st=None)) == OK


def test_pair_rejects(L):
    f = L.mx_quantize_pair
    X1, C1, S1 = P(0x60000000), P(0x70000000), P(0x78000000)
    args = lambda **k: [k.get("mode", 0), k.get("fmt", E4M3), 0,
                        k.get("x0", X), k.get("r0", 64), k.get("c0", 64), k.get("l0", 64), k.get("cd0", C),
                        k.get("s0", S), k.get("x1", X1), k.get("r1", 96), k.get("c1", 128), k.get("l1", 128),
                        k.get("cd1", C1), k.get("s1", S1), None]
    assert f(*args(mode=5)) == INVALID                   # unknown mode
    assert f(*args(mode=-1)) == INVALID
    assert f(*args(fmt=7)) == INVALID
    assert f(*args(c1=48, l1=48)) == INVALID             # row mode: cols % 32 of the second tensor
    assert f(*args(mode=1, r0=48)) == INVALID            # transposed modes: rows % 32
    assert f(*args(mode=2, r1=40)) == INVALID
    assert f(*args(l0=63)) == INVALID                    # ldx < cols
    assert f(*args(x1=None)) == INVALID
    assert f(*args(cd1=P(0x20000100))) == INVALID        # second codes inside the first codes
    assert f(*args(s1=P(0x30000010))) == INVALID         # second scales inside the first scales
    assert f(*args(cd0=P(0x60000000))) == INVALID        # first codes over the second input
    assert f(*args(s1=P(0x10000040))) == INVALID         # second scales over the first input
    assert f(*args(r0=0, r1=0, x0=None, x1=None, cd0=None, s0=None, cd1=None, s1=None)) == OK  # both empty
    # K-panel modes: rows a multiple of the panel width (128 FP8 elements, 256 E2M1)
    assert f(*args(mode=3, r0=128, r1=96)) == INVALID
    assert f(*args(mode=4, fmt=E2M1, r0=128, r1=256)) == INVALID
    assert f(*args(mode=4, fmt=E2M1, r0=256, r1=256, cd1=P(0x20000100))) == INVALID   # overlap still checked
    assert f(*args(mode=4, fmt=E2M1, r0=0, r1=0, x0=None, x1=None, cd0=None, s0=None, cd1=None, s1=None)) == OK


@pytest.mark.parametrize("fn", ["mx_quantize_transpose_panels", "mx_hadamard32_quantize_panels"])
def test_panel_quantize_rejects(L, fn):
    f = getattr(L, fn)
    rot = fn.startswith("mx_hadamard")
    call = lambda x, r, c, ld, fmt, cd, sc: f(x, r, c, ld, *((0, fmt) if rot else (fmt,)), cd, sc, None)
    assert call(X, 96, 4, 4, E4M3, C, S) == INVALID          # rows not a multiple of 128 (FP8 panel)
    assert call(X, 128, 4, 4, E2M1, C, S) == INVALID         # rows not a multiple of 256 (E2M1 panel)
    assert call(X, 128, 4, 4, 7, C, S) == INVALID            # format
    assert call(X, 128, 4, 3, E4M3, C, S) == INVALID         # ldx < cols
    assert call(X, 128, 4, 4, E4M3, X, S) == INVALID         # codes overlap x
    assert call(X, 128, 4, 4, E4M3, None, S) == INVALID
    assert call(None, 0, 4, 4, E4M3, None, None) == OK       # empty


def test_dual_panels_rejects(L):
    f = L.mx_quantize_dual_panels
    args = lambda **k: [k.get("x", X), k.get("rows", 256), k.get("cols", 256), k.get("ldx", 256), k.get("fr", E2M1),
                        k.get("cr", C), k.get("sr", S), k.get("ft", E2M1), k.get("rot", 1), 0, k.get("ct", C2),
                        k.get("st", S2), None]
    assert f(*args(cols=224, ldx=224)) == INVALID       # row form: cols not whole E2M1 panels
    assert f(*args(rows=128)) == INVALID                 # transposed form: rows not whole E2M1 panels
    assert f(*args(fr=E4M3, cols=320, ldx=320)) == INVALID   # not whole FP8 panels (128)
    assert f(*args(rot=2)) == INVALID
    assert f(*args(ct=C)) == INVALID                     # the two code buffers overlap
    assert f(*args(ft=9)) == INVALID
    assert f(*args(rows=0, x=None, cr=None, sr=None, ct=None, st=None)) == OK


def test_gemm_layout_rejects(L):
    f = L.mx_gemm_layout
    A, AS, B, BS, Cc = (P(a) for a in (0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000))
    ROWS, PANELS = 0, 1
    args = lambda **k: [k.get("a", A), k.get("la", PANELS), AS, k.get("fa", E2M1), k.get("b", B), k.get("lb", PANELS),
                        BS, k.get("fb", E2M1), k.get("M", 64), k.get("N", 64), k.get("K", 512), k.get("c", Cc), 0,
                        k.get("ldc", 64), None]
    assert f(*args(la=2)) == INVALID                           # unknown layout
    assert f(*args(lb=-1)) == INVALID
    assert f(*args(K=48)) == INVALID                           # mx_gemm's checks come first
    assert f(*args(ldc=63)) == INVALID
    assert f(*args(c=P(0x10000100))) == INVALID                # C overlaps A
    assert f(*args(K=256)) == UNSUPPORTED                      # panels need K % 512 == 0
    assert f(*args(a=P(0x10000008))) == UNSUPPORTED           # 16-byte aligned codes
    assert f(*args(fb=E4M3, lb=ROWS)) == UNSUPPORTED           # an E2M1 panel operand needs an E2M1 partner
    assert f(*args(M=1 << 23, K=1024, c=P(0x7000000000))) == UNSUPPORTED   # panel operand of 2^31 code bytes
    assert f(*args(M=0, a=None, c=None)) == OK                 # empty


def test_gemm_rejects(L):
    f = L.mx_gemm
    A, AS, B, BS, Cc = (P(a) for a in (0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000))
    assert f(A, AS, E4M3, B, BS, E4M3, 64, 64, 48, Cc, 0, 64, None) == INVALID   # K % 32
    assert f(A, AS, E4M3, B, BS, E4M3, -1, 64, 64, Cc, 0, 64, None) == INVALID
    assert f(A, AS, E4M3, B, BS, 3, 64, 64, 64, Cc, 0, 64, None) == INVALID     # format
    assert f(A, AS, E4M3, B, BS, E4M3, 64, 64, 64, Cc, 2, 64, None) == INVALID  # output type
    assert f(A, AS, E4M3, B, BS, E4M3, 64, 64, 64, Cc, 0, 63, None) == INVALID  # ldc < N
    assert f(A, AS, E4M3, B, BS, E4M3, 64, 64, 64, None, 0, 64, None) == INVALID
    assert f(None, AS, E4M3, B, BS, E4M3, 64, 64, 64, Cc, 0, 64, None) == INVALID
    assert f(A, AS, E4M3, B, BS, E4M3, 64, 64, 64, P(0x10000100), 0, 64, None) == INVALID  # C overlaps A
    assert f(None, None, E4M3, None, None, E4M3, 0, 64, 64, None, 0, 64, None) == OK       # empty


def test_quantize_strided_rejects(L):
    f = L.mx_quantize_strided
    # a payload of 64 rows x 4096 E4M3 elements: rows of [4096 code bytes | 128 scale bytes]
    PL = P(0x20000000)
    ok = lambda **k: [k.get("x", X), k.get("rows", 64), k.get("cols", 4096), k.get("ldx", 4096), k.get("fmt", E4M3),
                      k.get("c", PL), k.get("ldc", 4224), k.get("s", P(0x20000000 + 4096)), k.get("lds", 4224), None]
    assert f(*ok(cols=4008, ldx=4008)) == INVALID          # cols % 32
    assert f(*ok(ldc=4095)) == INVALID                     # code rows overlap each other
    assert f(*ok(lds=127)) == INVALID                      # scale row stride below cols / 32
    assert f(*ok(s=P(0x20000000 + 4000))) == INVALID       # scales inside the codes of their row
    assert f(*ok(s=P(0x20000000 + 4100))) == INVALID       # scales run into the next row's codes
    assert f(*ok(lds=4096 + 256)) == INVALID               # interleaved with a different stride
    assert f(*ok(x=P(0x20000100))) == INVALID              # input over the payload
    assert f(*ok(fmt=4)) == INVALID
    assert f(*ok(c=None)) == INVALID
    assert f(*ok(ldx=4095)) == INVALID
    assert f(*ok(rows=0, x=None, c=None, s=None)) == OK    # empty
    # E2M1 payload rows: 2048 code bytes + 128 scale bytes; misplaced scales are rejected
    assert f(*ok(fmt=E2M1, ldc=2176, lds=2176, s=P(0x20000000 + 2047))) == INVALID


def test_gemm_strided_rejects(L):
    f = L.mx_gemm_strided
    A, AS, B, BS, Cc = (P(a) for a in (0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000))
    args = lambda **k: [k.get("a", A), k.get("lda", 512), k.get("as_", AS), k.get("ldsa", 16), E4M3,
                        k.get("b", B), k.get("ldb", 512), k.get("bs", BS), k.get("ldsb", 16), k.get("fb", E2M1),
                        k.get("M", 64), k.get("N", 64), k.get("K", 512), k.get("c", Cc), 0, k.get("ldc", 64), None]
    assert f(*args(lda=511)) == INVALID                  # code row stride below K bytes (E4M3)
    assert f(*args(lda=520)) == INVALID                  # code row stride not a multiple of 16
    assert f(*args(ldb=255)) == INVALID                  # below K / 2 (E2M1)
    assert f(*args(ldsa=15)) == INVALID                  # scale row stride below K / 32
    assert f(*args(ldsb=15)) == INVALID
    assert f(*args(K=500)) == INVALID
    assert f(*args(ldc=63)) == INVALID
    assert f(*args(c=P(0x10000000 + 63 * 512))) == INVALID   # C over A's last row (strided extent)
    assert f(*args(c=P(0x20000000 + 63 * 16))) == INVALID    # C over A's last scale row
    assert f(*args(M=0, a=None, as_=None, c=None)) == OK     # empty


def test_valid_call_without_a_device_reports_hip_error(L):
    """past validation the library asks HIP for the device; without one it
    returns MX_ERR_HIP instead of crashing (with a GPU present this would
    launch, so it is skipped there)"""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; the launch path is covered by the GPU tests")
    assert L.mx_quantize(X, 4, 64, 64, E4M3, C, S, None) == HIPERR
