// mx_api.hip -- the extern "C" entry points declared in include/mx.h.
//
// Every argument is validated on the host before the first HIP call, so the
// error paths run (and are tested) without a GPU.  After validation the
// current device is checked to be gfx950 (once per device, cached) and the
// kernels are launched on the caller's stream.  Nothing is allocated and no
// call synchronizes.
#include <atomic>
#include <string.h>

#include "mx.h"
#include "mx_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

// An enum parameter's value as the caller passed it.  A C caller may pass any
// int through an enum type, but in C++ a load of an enum object whose value
// lies outside its enumerators' range has no defined meaning; the entry
// points therefore read their enum parameters' bytes as an int and validate
// that.
template <class E>
int raw(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "the ABI's enums are int-sized");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}

bool fmt_ok(int f) { return f == MX_E4M3 || f == MX_E5M2 || f == MX_E2M1; }

int64_t code_bytes(int64_t n, int fmt) { return fmt == MX_E2M1 ? n / 2 : n; }

// K-panel width in elements: 128 code bytes
int64_t panel_elems(int fmt) { return fmt == MX_E2M1 ? 256 : 128; }

// half-open byte ranges [p, p + n) overlap
bool overlap(const void *p, int64_t n, const void *q, int64_t m) {
    if (n <= 0 || m <= 0) return false;
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

mx_status_t check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MX_ERR_HIP;
    if (dev >= kMaxDevices) return MX_ERR_UNSUPPORTED;
    int st = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MX_ERR_HIP;
        st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_ok[dev].store(st, std::memory_order_relaxed);
    }
    return st == 1 ? MX_OK : MX_ERR_UNSUPPORTED;
}

// shared checks of the three quantizers; `blocked` is the dimension cut into
// 32-element blocks (cols in row mode, rows in transposed mode)
mx_status_t check_quant(const void *x, int64_t rows, int64_t cols, int64_t ldx, int fmt, const void *codes,
                        const void *scales, bool transposed) {
    if (rows < 0 || cols < 0 || !fmt_ok(fmt)) return MX_ERR_INVALID_ARG;
    const int64_t blocked = transposed ? rows : cols;
    if (blocked % 32 != 0) return MX_ERR_INVALID_ARG;
    if (ldx < cols) return MX_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return MX_OK;
    if (!x || !codes || !scales) return MX_ERR_INVALID_ARG;
    // index ranges the kernels address in 32 bits: octets (row mode), rows, columns
    if (rows > (int64_t)1 << 31 || cols > (int64_t)1 << 31) return MX_ERR_UNSUPPORTED;
    if (rows > INT64_MAX / ldx) return MX_ERR_INVALID_ARG;
    const int64_t n = rows * cols;
    if (!transposed && n / 8 >= ((int64_t)1 << 32)) return MX_ERR_UNSUPPORTED;
    const int64_t xb = ((rows - 1) * ldx + cols) * 2;
    const int64_t cb = code_bytes(n, fmt), sb = n / 32;
    if (overlap(x, xb, codes, cb) || overlap(x, xb, scales, sb) || overlap(codes, cb, scales, sb))
        return MX_ERR_INVALID_ARG;
    return MX_OK;
}

mx_status_t launched(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

// Two strided row patterns, `rows` rows each: row i of the first covers bytes
// [p + i * lp, p + i * lp + wp), row j of the second [q + j * lq, q + j * lq + wq).
// They are disjoint if their whole extents are, or if they share one stride L
// and, within every period of L bytes, the second's row sits in the gap after
// the first's (the layout of rows of [codes | scales] in one buffer).
bool strided_overlap(const void *p, int64_t lp, int64_t wp, const void *q, int64_t lq, int64_t wq, int64_t rows) {
    if (rows <= 0 || wp <= 0 || wq <= 0) return false;
    if (!overlap(p, (rows - 1) * lp + wp, q, (rows - 1) * lq + wq)) return false;
    if (lp != lq) return true;
    const int64_t L = lp;
    int64_t d = (int64_t)((uintptr_t)q - (uintptr_t)p) % L;
    if (d < 0) d += L;
    return !(d >= wp && d + wq <= L);
}

// checks of the GEMM's arguments, operand row strides in bytes
mx_status_t check_gemm(const void *a_codes, int64_t lda, const void *a_scales, int64_t ldsa, int fa,
                       const void *b_codes, int64_t ldb, const void *b_scales, int64_t ldsb, int fb, int64_t M,
                       int64_t N, int64_t K, const void *c, int out, int64_t ldc) {
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return MX_ERR_INVALID_ARG;
    if (!fmt_ok(fa) || !fmt_ok(fb) || (out != MX_OUT_F32 && out != MX_OUT_BF16)) return MX_ERR_INVALID_ARG;
    if (ldc < N) return MX_ERR_INVALID_ARG;
    if (lda < code_bytes(K, fa) || ldb < code_bytes(K, fb) || ldsa < K / 32 || ldsb < K / 32)
        return MX_ERR_INVALID_ARG;
    // code rows are read with 16-byte loads (dense rows always qualify: K % 32 == 0)
    if (lda % 16 != 0 || ldb % 16 != 0) return MX_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return MX_OK;
    if (!c) return MX_ERR_INVALID_ARG;
    if (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales)) return MX_ERR_INVALID_ARG;
    if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31))
        return MX_ERR_UNSUPPORTED;
    if ((M + 255) / 256 * ((N + 255) / 256) >= ((int64_t)1 << 31)) return MX_ERR_UNSUPPORTED;
    if (M - 1 > (INT64_MAX - N) / ldc) return MX_ERR_INVALID_ARG;
    if (K > 0 && ((M - 1) > INT64_MAX / lda || (N - 1) > INT64_MAX / ldb || (M - 1) > INT64_MAX / ldsa ||
                  (N - 1) > INT64_MAX / ldsb))
        return MX_ERR_INVALID_ARG;
    const int64_t cbytes = ((M - 1) * ldc + N) * (out == MX_OUT_BF16 ? 2 : 4);
    if (K > 0) {
        const int64_t ab = (M - 1) * lda + code_bytes(K, fa), bb = (N - 1) * ldb + code_bytes(K, fb);
        const int64_t asb = (M - 1) * ldsa + K / 32, bsb = (N - 1) * ldsb + K / 32;
        if (overlap(c, cbytes, a_codes, ab) || overlap(c, cbytes, a_scales, asb) ||
            overlap(c, cbytes, b_codes, bb) || overlap(c, cbytes, b_scales, bsb))
            return MX_ERR_INVALID_ARG;
    }
    return MX_OK;
}

// mx_gemm_strided with its enum arguments already read as ints
mx_status_t gemm_strided(const void *a_codes, int64_t lda, const void *a_scales, int64_t ldsa, int fa,
                         const void *b_codes, int64_t ldb, const void *b_scales, int64_t ldsb, int fb, int64_t M,
                         int64_t N, int64_t K, void *c, int out, int64_t ldc, void *stream, int64_t kpa = 0,
                         int64_t kpb = 0) {
    mx_status_t st = check_gemm(a_codes, lda, a_scales, ldsa, fa, b_codes, ldb, b_scales, ldsb, fb, M, N, K, c, out,
                                ldc);
    if (st != MX_OK || M == 0 || N == 0) return st;
    if ((st = check_device()) != MX_OK) return st;
    return launched(mx::launch_gemm((const uint8_t *)a_codes, lda, (const uint8_t *)a_scales, ldsa, fa,
                                    (const uint8_t *)b_codes, ldb, (const uint8_t *)b_scales, ldsb, fb, M, N, K, c,
                                    out == MX_OUT_BF16, ldc, (hipStream_t)stream, kpa, kpb));
}

// the transposed quantizers with K-panel code output
mx_status_t quantize_transpose_panels(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx, int f,
                                      bool rotate, uint32_t sign_mask, void *codes, void *scales, void *stream) {
    mx_status_t st = check_quant(x_bf16, rows, cols, ldx, f, codes, scales, true);
    if (st != MX_OK) return st;
    if (rows % panel_elems(f) != 0) return MX_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return MX_OK;
    if ((st = check_device()) != MX_OK) return st;
    return launched(mx::launch_quantize_transpose((const uint16_t *)x_bf16, rows, cols, ldx, f, rotate, sign_mask,
                                                  (uint8_t *)codes, (uint8_t *)scales, (hipStream_t)stream, true));
}

// the fused dual-direction quantizer, with row-major or K-panel code outputs
mx_status_t quantize_dual(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx, int fr, void *codes_row,
                          void *scales_row, int ft, int rotate, uint32_t sign_mask, void *codes_t, void *scales_t,
                          void *stream, bool panels) {
    if (rotate != 0 && rotate != 1) return MX_ERR_INVALID_ARG;
    // K-panel outputs: each form's K (cols for the row form, rows for the transposed one) whole panels
    if (panels && fmt_ok(fr) && fmt_ok(ft) && (cols % panel_elems(fr) != 0 || rows % panel_elems(ft) != 0))
        return MX_ERR_INVALID_ARG;
    mx_status_t st = check_quant(x_bf16, rows, cols, ldx, fr, codes_row, scales_row, false);
    if (st != MX_OK) return st;
    if ((st = check_quant(x_bf16, rows, cols, ldx, ft, codes_t, scales_t, true)) != MX_OK) return st;
    if (rows == 0 || cols == 0) return MX_OK;
    const int64_t n = rows * cols;
    const int64_t crb = code_bytes(n, fr), ctb = code_bytes(n, ft), sb = n / 32;
    if (overlap(codes_row, crb, codes_t, ctb) || overlap(codes_row, crb, scales_t, sb) ||
        overlap(scales_row, sb, codes_t, ctb) || overlap(scales_row, sb, scales_t, sb))
        return MX_ERR_INVALID_ARG;
    if ((st = check_device()) != MX_OK) return st;
    return launched(mx::launch_quantize_dual((const uint16_t *)x_bf16, rows, cols, ldx, fr, (uint8_t *)codes_row,
                                             (uint8_t *)scales_row, ft, rotate != 0, sign_mask, (uint8_t *)codes_t,
                                             (uint8_t *)scales_t, (hipStream_t)stream, panels));
}

}  // namespace

extern "C" {

const char *mx_status_string(mx_status_t s) {
    switch (raw(s)) {
    case MX_OK: return "MX_OK";
    case MX_ERR_INVALID_ARG: return "MX_ERR_INVALID_ARG";
    case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
    case MX_ERR_HIP: return "MX_ERR_HIP";
    }
    return "MX_ERR_UNKNOWN";
}

int mx_version(void) { return 100; }

mx_status_t mx_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx, mx_format_t fmt,
                        void *codes, void *scales, void *stream) {
    const int f = raw(fmt);
    mx_status_t st = check_quant(x_bf16, rows, cols, ldx, f, codes, scales, false);
    if (st != MX_OK || rows == 0 || cols == 0) return st;
    if ((st = check_device()) != MX_OK) return st;
    return launched(mx::launch_quantize_rows((const uint16_t *)x_bf16, rows, cols, ldx, f, (uint8_t *)codes,
                                             (uint8_t *)scales, (hipStream_t)stream));
}

mx_status_t mx_quantize_transpose(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                                  mx_format_t fmt, void *codes, void *scales, void *stream) {
    const int f = raw(fmt);
    mx_status_t st = check_quant(x_bf16, rows, cols, ldx, f, codes, scales, true);
    if (st != MX_OK || rows == 0 || cols == 0) return st;
    if ((st = check_device()) != MX_OK) return st;
    return launched(mx::launch_quantize_transpose((const uint16_t *)x_bf16, rows, cols, ldx, f, false, 0,
                                                  (uint8_t *)codes, (uint8_t *)scales, (hipStream_t)stream));
}

mx_status_t mx_hadamard32_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                                   uint32_t sign_mask, mx_format_t fmt, void *codes, void *scales,
                                   void *stream) {
    const int f = raw(fmt);
    mx_status_t st = check_quant(x_bf16, rows, cols, ldx, f, codes, scales, true);
    if (st != MX_OK || rows == 0 || cols == 0) return st;
    if ((st = check_device()) != MX_OK) return st;
    return launched(mx::launch_quantize_transpose((const uint16_t *)x_bf16, rows, cols, ldx, f, true,
                                                  sign_mask, (uint8_t *)codes, (uint8_t *)scales,
                                                  (hipStream_t)stream));
}

mx_status_t mx_quantize_transpose_panels(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                                         mx_format_t fmt, void *codes, void *scales, void *stream) {
    return quantize_transpose_panels(x_bf16, rows, cols, ldx, raw(fmt), false, 0u, codes, scales, stream);
}

mx_status_t mx_hadamard32_quantize_panels(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                                          uint32_t sign_mask, mx_format_t fmt, void *codes, void *scales,
                                          void *stream) {
    return quantize_transpose_panels(x_bf16, rows, cols, ldx, raw(fmt), true, sign_mask, codes, scales, stream);
}

mx_status_t mx_quantize_transpose_sr(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx, int rotate,
                                     uint32_t sign_mask, uint64_t seed, mx_format_t fmt, void *codes, void *scales,
                                     void *stream) {
    const int f = raw(fmt);
    if (rotate != 0 && rotate != 1) return MX_ERR_INVALID_ARG;
    mx_status_t st = check_quant(x_bf16, rows, cols, ldx, f, codes, scales, true);
    if (st != MX_OK || rows == 0 || cols == 0) return st;
    if ((st = check_device()) != MX_OK) return st;
    return launched(mx::launch_quantize_transpose_sr((const uint16_t *)x_bf16, rows, cols, ldx, f, rotate != 0,
                                                     sign_mask, seed, (uint8_t *)codes, (uint8_t *)scales,
                                                     (hipStream_t)stream));
}

mx_status_t mx_quantize_dual(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx, mx_format_t fmt_row,
                             void *codes_row, void *scales_row, mx_format_t fmt_t, int rotate, uint32_t sign_mask,
                             void *codes_t, void *scales_t, void *stream) {
    return quantize_dual(x_bf16, rows, cols, ldx, raw(fmt_row), codes_row, scales_row, raw(fmt_t), rotate, sign_mask,
                         codes_t, scales_t, stream, false);
}

mx_status_t mx_quantize_dual_panels(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx, mx_format_t fmt_row,
                                    void *codes_row, void *scales_row, mx_format_t fmt_t, int rotate,
                                    uint32_t sign_mask, void *codes_t, void *scales_t, void *stream) {
    return quantize_dual(x_bf16, rows, cols, ldx, raw(fmt_row), codes_row, scales_row, raw(fmt_t), rotate, sign_mask,
                         codes_t, scales_t, stream, true);
}

mx_status_t mx_quantize_pair(mx_pair_mode_t mode, mx_format_t fmt, uint32_t sign_mask, const void *x0,
                             int64_t rows0, int64_t cols0, int64_t ldx0, void *codes0, void *scales0, const void *x1,
                             int64_t rows1, int64_t cols1, int64_t ldx1, void *codes1, void *scales1, void *stream) {
    const int m = raw(mode);
    const int f = raw(fmt);
    if (m != MX_PAIR_ROW && m != MX_PAIR_TRANSPOSE && m != MX_PAIR_HADAMARD && m != MX_PAIR_TRANSPOSE_PANELS &&
        m != MX_PAIR_HADAMARD_PANELS)
        return MX_ERR_INVALID_ARG;
    const bool tr = m != MX_PAIR_ROW;
    const bool panels = m == MX_PAIR_TRANSPOSE_PANELS || m == MX_PAIR_HADAMARD_PANELS;
    const bool rot = m == MX_PAIR_HADAMARD || m == MX_PAIR_HADAMARD_PANELS;
    if (panels && fmt_ok(f) && (rows0 % panel_elems(f) != 0 || rows1 % panel_elems(f) != 0))
        return MX_ERR_INVALID_ARG;
    mx_status_t st = check_quant(x0, rows0, cols0, ldx0, f, codes0, scales0, tr);
    if (st != MX_OK) return st;
    if ((st = check_quant(x1, rows1, cols1, ldx1, f, codes1, scales1, tr)) != MX_OK) return st;
    const bool e0 = rows0 == 0 || cols0 == 0, e1 = rows1 == 0 || cols1 == 0;
    if (e0 && e1) return MX_OK;
    if (!e0 && !e1) {
        // no output of one tensor may overlap the other tensor's input or outputs
        const int64_t n0 = rows0 * cols0, n1 = rows1 * cols1;
        const int64_t xb0 = ((rows0 - 1) * ldx0 + cols0) * 2, xb1 = ((rows1 - 1) * ldx1 + cols1) * 2;
        const int64_t cb0 = code_bytes(n0, f), cb1 = code_bytes(n1, f), sb0 = n0 / 32, sb1 = n1 / 32;
        if (overlap(codes0, cb0, x1, xb1) || overlap(codes0, cb0, codes1, cb1) || overlap(codes0, cb0, scales1, sb1) ||
            overlap(scales0, sb0, x1, xb1) || overlap(scales0, sb0, codes1, cb1) || overlap(scales0, sb0, scales1, sb1) ||
            overlap(codes1, cb1, x0, xb0) || overlap(scales1, sb1, x0, xb0))
            return MX_ERR_INVALID_ARG;
    }
    if ((st = check_device()) != MX_OK) return st;
    const hipStream_t s = (hipStream_t)stream;
    const mx::QuantJob j0{(const uint16_t *)x0, rows0, cols0, ldx0, (uint8_t *)codes0, (uint8_t *)scales0};
    const mx::QuantJob j1{(const uint16_t *)x1, rows1, cols1, ldx1, (uint8_t *)codes1, (uint8_t *)scales1};
    if (e0 || e1) {  // one tensor: the single call
        const mx::QuantJob &j = e0 ? j1 : j0;
        if (!tr) return launched(mx::launch_quantize_rows(j.x, j.rows, j.cols, j.ldx, f, j.codes, j.scales, s));
        return launched(mx::launch_quantize_transpose(j.x, j.rows, j.cols, j.ldx, f, rot, rot ? sign_mask : 0u,
                                                      j.codes, j.scales, s, panels));
    }
    return launched(mx::launch_quantize_pair(m, f, rot ? sign_mask : 0u, j0, j1, s));
}

mx_status_t mx_gemm(const void *a_codes, const void *a_scales, mx_format_t fa, const void *b_codes,
                    const void *b_scales, mx_format_t fb, int64_t M, int64_t N, int64_t K, void *c,
                    mx_out_t out, int64_t ldc, void *stream) {
    const int a = raw(fa), b = raw(fb);
    if (!fmt_ok(a) || !fmt_ok(b) || K < 0) return MX_ERR_INVALID_ARG;
    return gemm_strided(a_codes, code_bytes(K, a), a_scales, K / 32, a, b_codes, code_bytes(K, b), b_scales, K / 32,
                        b, M, N, K, c, raw(out), ldc, stream);
}

mx_status_t mx_gemm_strided(const void *a_codes, int64_t lda, const void *a_scales, int64_t ldsa, mx_format_t fa,
                            const void *b_codes, int64_t ldb, const void *b_scales, int64_t ldsb, mx_format_t fb,
                            int64_t M, int64_t N, int64_t K, void *c, mx_out_t out, int64_t ldc, void *stream) {
    return gemm_strided(a_codes, lda, a_scales, ldsa, raw(fa), b_codes, ldb, b_scales, ldsb, raw(fb), M, N, K, c,
                        raw(out), ldc, stream);
}

mx_status_t mx_gemm_layout(const void *a_codes, mx_layout_t a_layout, const void *a_scales, mx_format_t fa,
                           const void *b_codes, mx_layout_t b_layout, const void *b_scales, mx_format_t fb,
                           int64_t M, int64_t N, int64_t K, void *c, mx_out_t out, int64_t ldc, void *stream) {
    const int a = raw(fa), b = raw(fb), la = raw(a_layout), lb = raw(b_layout);
    if (!fmt_ok(a) || !fmt_ok(b) || K < 0 || (la != MX_LAYOUT_ROWS && la != MX_LAYOUT_PANELS) ||
        (lb != MX_LAYOUT_ROWS && lb != MX_LAYOUT_PANELS))
        return MX_ERR_INVALID_ARG;
    const int64_t lda = code_bytes(K, a), ldb = code_bytes(K, b);
    int64_t kpa = 0, kpb = 0;
    if (la == MX_LAYOUT_PANELS || lb == MX_LAYOUT_PANELS) {
        // the argument checks of mx_gemm first (their errors take precedence)
        mx_status_t st = check_gemm(a_codes, lda, a_scales, K / 32, a, b_codes, ldb, b_scales, K / 32, b, M, N, K, c,
                                    raw(out), ldc);
        if (st != MX_OK || M == 0 || N == 0) return st;
        const bool fp4 = a == MX_E2M1 && b == MX_E2M1;
        const bool aligned = ((uintptr_t)a_codes % 16 == 0) && ((uintptr_t)b_codes % 16 == 0) &&
                             ((uintptr_t)a_scales % 4 == 0) && ((uintptr_t)b_scales % 4 == 0);
        if (K % 512 != 0 || !aligned) return MX_ERR_UNSUPPORTED;
        if (la == MX_LAYOUT_PANELS) {
            if ((a == MX_E2M1 && !fp4) || M * lda >= ((int64_t)1 << 31)) return MX_ERR_UNSUPPORTED;
            kpa = M * 128;
        }
        if (lb == MX_LAYOUT_PANELS) {
            if ((b == MX_E2M1 && !fp4) || N * ldb >= ((int64_t)1 << 31)) return MX_ERR_UNSUPPORTED;
            kpb = N * 128;
        }
    }
    return gemm_strided(a_codes, lda, a_scales, K / 32, a, b_codes, ldb, b_scales, K / 32, b, M, N, K, c, raw(out),
                        ldc, stream, kpa, kpb);
}

mx_status_t mx_quantize_strided(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx, mx_format_t fmt,
                                void *codes, int64_t ld_codes, void *scales, int64_t ld_scales, void *stream) {
    const int f = raw(fmt);
    if (rows < 0 || cols < 0 || !fmt_ok(f) || cols % 32 != 0 || ldx < cols) return MX_ERR_INVALID_ARG;
    const int64_t cbr = code_bytes(cols, f), sbr = cols / 32;
    if (ld_codes < cbr || ld_scales < sbr) return MX_ERR_INVALID_ARG;
    if (rows == 0 || cols == 0) return MX_OK;
    if (!x_bf16 || !codes || !scales) return MX_ERR_INVALID_ARG;
    if (rows > (int64_t)1 << 31 || cols > (int64_t)1 << 31) return MX_ERR_UNSUPPORTED;
    if (rows > INT64_MAX / ldx || rows > INT64_MAX / ld_codes || rows > INT64_MAX / ld_scales)
        return MX_ERR_INVALID_ARG;
    if ((rows * cols) / 8 >= ((int64_t)1 << 32)) return MX_ERR_UNSUPPORTED;
    const int64_t xb = ((rows - 1) * ldx + cols) * 2;
    if (overlap(x_bf16, xb, codes, (rows - 1) * ld_codes + cbr) || overlap(x_bf16, xb, scales, (rows - 1) * ld_scales + sbr) ||
        strided_overlap(codes, ld_codes, cbr, scales, ld_scales, sbr, rows))
        return MX_ERR_INVALID_ARG;
    mx_status_t st = check_device();
    if (st != MX_OK) return st;
    return launched(mx::launch_quantize_rows_strided((const uint16_t *)x_bf16, rows, cols, ldx, f, (uint8_t *)codes,
                                                     ld_codes, (uint8_t *)scales, ld_scales, (hipStream_t)stream));
}

}  // extern "C"
