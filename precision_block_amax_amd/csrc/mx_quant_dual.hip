// mx_quant_dual.hip -- launcher of the fused dual-direction quantizer: one
// read of a bf16 matrix yields its row MX form (the Fprop / Dgrad operand)
// and its transposed MX form, optionally after the fixed-sign block rotation
// (the weight-gradient operand).  Both forms are bit-identical to
// mx_quantize and to mx_quantize_transpose / mx_hadamard32_quantize.  The
// kernel is the transposed quantizer of mx_quant_kernels.h with its row-form
// output switched on; it saves one read of the input (2 bytes per element).
#include "mx_quant_kernels.h"

namespace mx {
namespace {

template <int FR, int FT, bool ROTATE>
hipError_t launch_dual_fmt(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, uint32_t mask,
                           uint8_t *codes_r, uint8_t *scales_r, uint8_t *codes_t, uint8_t *scales_t,
                           hipStream_t stream, bool panels) {
    const bool vec = ((uintptr_t)x % 8 == 0) && (ldx % 4 == 0) && ((uintptr_t)codes_t % 16 == 0) &&
                     ((uintptr_t)codes_r % 16 == 0);
    constexpr int W = tr_waves<FT, true, FR, false>();
    static_assert(W == tr_waves<FT, false, FR, false>(), "one grid for both variants");
    const dim3 grid((unsigned)((cols + kTrCols - 1) / kTrCols), (unsigned)((rows / 32 + W - 1) / W));
    if (vec)
        hipLaunchKernelGGL((k_quantize_transpose<FT, ROTATE, true, FR>), grid, dim3(64 * W), 0, stream, x,
                           ldx, rows, cols, mask, codes_t, scales_t, codes_r, scales_r, (uint64_t)0, nullptr, 0, 0, 0,
                           nullptr, nullptr, 0u, panels ? 1 : 0);
    else
        hipLaunchKernelGGL((k_quantize_transpose<FT, ROTATE, false, FR>), grid, dim3(64 * W), 0, stream, x,
                           ldx, rows, cols, mask, codes_t, scales_t, codes_r, scales_r, (uint64_t)0, nullptr, 0, 0, 0,
                           nullptr, nullptr, 0u, panels ? 1 : 0);
    return hipGetLastError();
}

template <int FR, bool ROTATE>
hipError_t launch_dual_t(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt_t, uint32_t mask,
                         uint8_t *cr, uint8_t *sr, uint8_t *ct, uint8_t *st, hipStream_t s, bool p) {
    switch (fmt_t) {
    case E4M3: return launch_dual_fmt<FR, E4M3, ROTATE>(x, rows, cols, ldx, mask, cr, sr, ct, st, s, p);
    case E5M2: return launch_dual_fmt<FR, E5M2, ROTATE>(x, rows, cols, ldx, mask, cr, sr, ct, st, s, p);
    default: return launch_dual_fmt<FR, E2M1, ROTATE>(x, rows, cols, ldx, mask, cr, sr, ct, st, s, p);
    }
}

template <bool ROTATE>
hipError_t launch_dual_r(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt_r, int fmt_t,
                         uint32_t mask, uint8_t *cr, uint8_t *sr, uint8_t *ct, uint8_t *st, hipStream_t s, bool p) {
    switch (fmt_r) {
    case E4M3: return launch_dual_t<E4M3, ROTATE>(x, rows, cols, ldx, fmt_t, mask, cr, sr, ct, st, s, p);
    case E5M2: return launch_dual_t<E5M2, ROTATE>(x, rows, cols, ldx, fmt_t, mask, cr, sr, ct, st, s, p);
    default: return launch_dual_t<E2M1, ROTATE>(x, rows, cols, ldx, fmt_t, mask, cr, sr, ct, st, s, p);
    }
}

}  // namespace

hipError_t launch_quantize_dual(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt_r,
                                uint8_t *codes_r, uint8_t *scales_r, int fmt_t, bool rotate, uint32_t sign_mask,
                                uint8_t *codes_t, uint8_t *scales_t, hipStream_t stream, bool panels) {
    if (rotate)
        return launch_dual_r<true>(x, rows, cols, ldx, fmt_r, fmt_t, sign_mask, codes_r, scales_r, codes_t, scales_t,
                                   stream, panels);
    return launch_dual_r<false>(x, rows, cols, ldx, fmt_r, fmt_t, 0, codes_r, scales_r, codes_t, scales_t, stream,
                                panels);
}

}  // namespace mx
