// mx_internal.h -- launchers and small device utilities shared by the libmx
// translation units.  Not part of the public ABI (include/mx.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_convert.h"

namespace mx {

// Unsigned 32-bit division by a runtime-constant divisor d >= 1 as a
// multiply-high and shift (Granlund & Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l for every
// 32-bit n (the add is done in 64 bits).
struct FastDiv {
    uint32_t d, m, l;
    MXHD FastDiv() : d(1), m(1), l(0) {}
    explicit FastDiv(uint32_t div) : d(div) {
        l = 0;
        while ((1ull << l) < div) l++;
        m = (uint32_t)((((1ull << l) - div) << 32) / div + 1);
    }
    MXHD uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
        uint32_t hi = __umulhi(m, n);
#else
        uint32_t hi = (uint32_t)(((uint64_t)m * n) >> 32);
#endif
        return (uint32_t)(((uint64_t)hi + n) >> l);
    }
};

// Quantize launchers (mx_quant.hip).  All sizes validated by the caller;
// they return the launch status.
hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                uint8_t *codes, uint8_t *scales, hipStream_t stream);
hipError_t launch_quantize_transpose(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                                     int fmt, bool rotate, uint32_t sign_mask, uint8_t *codes,
                                     uint8_t *scales, hipStream_t stream, bool panels = false);

// transposed mode (rotated or not) with stochastic rounding under `seed`
hipError_t launch_quantize_transpose_sr(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                        bool rotate, uint32_t sign_mask, uint64_t seed, uint8_t *codes,
                                        uint8_t *scales, hipStream_t stream);

// one read of x: row form (fmt_r) and transposed form (fmt_t, rotated or not)
hipError_t launch_quantize_dual(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt_r,
                                uint8_t *codes_r, uint8_t *scales_r, int fmt_t, bool rotate, uint32_t sign_mask,
                                uint8_t *codes_t, uint8_t *scales_t, hipStream_t stream, bool panels = false);

// one tensor of a pair quantization: bf16 input [rows x ldx], outputs as the single call's
struct QuantJob {
    const uint16_t *x;
    int64_t rows, cols, ldx;
    uint8_t *codes, *scales;
};

// Both tensors in one launch (mode 0: row, 1: transposed, 2: rotated transposed, 3 and 4:
// modes 1 and 2 with K-panel code output), or two launches where they need different
// kernel variants.  Both non-empty.
hipError_t launch_quantize_pair(int mode, int fmt, uint32_t sign_mask, const QuantJob &a, const QuantJob &b,
                                hipStream_t stream);

// GEMM launcher (mx_gemm.hip); operand row strides in bytes (codes, scales);
// kpa / kpb != 0: that operand's codes are K-panel-major with this panel
// stride in bytes (GemmArgs).
hipError_t launch_gemm(const uint8_t *a, int64_t lda, const uint8_t *as, int64_t ldsa, int fa, const uint8_t *b,
                       int64_t ldb, const uint8_t *bs, int64_t ldsb, int fb, int64_t M, int64_t N, int64_t K, void *c,
                       bool bf16_out, int64_t ldc, hipStream_t stream, int64_t kpa = 0, int64_t kpb = 0);

// Row mode with strided outputs: row r's codes at codes + r * ld_codes, its
// scales at scales + r * ld_scales (bytes).
hipError_t launch_quantize_rows_strided(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                        uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                                        hipStream_t stream);

}  // namespace mx
