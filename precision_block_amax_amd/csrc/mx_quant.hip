// mx_quant.hip -- MX quantizers for gfx950: row mode, transposed mode, and
// transposed mode after the fixed-sign 32-point block-Hadamard rotation.
//
// Method: MX micro-scaling, block 32 along the reduction dimension, E8M0
// scale from the block amax, round-to-nearest-even saturating element casts
// (FP4-training article on hzrcw.cc, section 02; MindSpeed-LLM FSDP2 page,
// recipe dynamic_MX-1-1-32); the rotation is the deterministic Hadamard
// transform that article applies on the weight-gradient path.  Element and
// scale arithmetic is in mx_convert.h.
//
// All three kernels are HBM-bandwidth bound (2 B read + 1 or 0.5 B written +
// 1/32 B of scale per element).  Design:
//   row mode   each lane holds 8 consecutive bf16 (one 16-byte load), four
//              neighbouring lanes form a 32-element block, the block amax is a
//              two-step DPP quad reduction; every load and store instruction
//              of a wave covers one contiguous span.
//   transposed each lane holds 4 adjacent columns of a 32-row block (32
//              8-byte loads, each wave instruction reading 512 contiguous
//              bytes of one row), so a whole block sits in one lane's
//              registers: amax and, for the rotation, the five butterfly
//              stages need no cross-lane traffic.  A workgroup covers 8 row
//              blocks; its codes are staged in LDS and stored as whole
//              128-byte (E2M1) or 256-byte (FP8) runs of each output row, since
//              one 16-byte store per lane and output row wrote at about a
//              third of the read rate.
#include "mx_quant_kernels.h"

namespace mx {
namespace {

template <int F>
hipError_t launch_rows_fmt(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, uint8_t *codes,
                           uint8_t *scales, hipStream_t stream) {
    const uint64_t total = (uint64_t)rows * (uint64_t)cols / 8;
    const uint32_t opr = (uint32_t)(cols / 8);
    const bool contig = ldx == cols;
    const bool vec = ((uintptr_t)x % 16 == 0) && (ldx % 8 == 0) &&
                     ((uintptr_t)codes % (F == E2M1 ? 4 : 8) == 0);
    const uint32_t per_block = kRowThreads * kRowUnroll;
    const dim3 grid((unsigned)((total + per_block - 1) / per_block));
    const FastDiv div(opr);
    if (contig && vec)
        hipLaunchKernelGGL((k_quantize_rows<F, true, true>), grid, dim3(kRowThreads), 0, stream, x, ldx,
                           (uint32_t)total, opr, div, codes, scales);
    else if (vec)
        hipLaunchKernelGGL((k_quantize_rows<F, false, true>), grid, dim3(kRowThreads), 0, stream, x, ldx,
                           (uint32_t)total, opr, div, codes, scales);
    else
        hipLaunchKernelGGL((k_quantize_rows<F, false, false>), grid, dim3(kRowThreads), 0, stream, x, ldx,
                           (uint32_t)total, opr, div, codes, scales);
    return hipGetLastError();
}

// strided outputs (OSTR): the row index comes from the octet index in both
// input layouts, so only the non-contiguous input variants are instantiated
template <int F>
hipError_t launch_rows_strided_fmt(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, uint8_t *codes,
                                   int64_t ld_codes, uint8_t *scales, int64_t ld_scales, hipStream_t stream) {
    const uint64_t total = (uint64_t)rows * (uint64_t)cols / 8;
    const uint32_t opr = (uint32_t)(cols / 8);
    constexpr int CB = F == E2M1 ? 4 : 8;
    const bool vec = ((uintptr_t)x % 16 == 0) && (ldx % 8 == 0) && ((uintptr_t)codes % CB == 0) && (ld_codes % CB == 0);
    const uint32_t per_block = kRowThreads * kRowUnroll;
    const dim3 grid((unsigned)((total + per_block - 1) / per_block));
    const FastDiv div(opr);
    if (vec)
        hipLaunchKernelGGL((k_quantize_rows<F, false, true, false, true>), grid, dim3(kRowThreads), 0, stream, x, ldx,
                           (uint32_t)total, opr, div, codes, scales, nullptr, 0, 0u, 0u, FastDiv(), nullptr, nullptr,
                           0u, ld_codes, ld_scales);
    else
        hipLaunchKernelGGL((k_quantize_rows<F, false, false, false, true>), grid, dim3(kRowThreads), 0, stream, x, ldx,
                           (uint32_t)total, opr, div, codes, scales, nullptr, 0, 0u, 0u, FastDiv(), nullptr, nullptr,
                           0u, ld_codes, ld_scales);
    return hipGetLastError();
}

template <int F, bool ROTATE>
hipError_t launch_tr_fmt(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, uint32_t mask,
                         uint8_t *codes, uint8_t *scales, hipStream_t stream, bool panels = false) {
    const bool vec = ((uintptr_t)x % 8 == 0) && (ldx % 4 == 0) && ((uintptr_t)codes % 16 == 0);
    const unsigned tx = (unsigned)((cols + kTrCols - 1) / kTrCols);
    if (vec) {
        constexpr int W = tr_waves<F, true, -1, false>();
        hipLaunchKernelGGL((k_quantize_transpose<F, ROTATE, true>), dim3(tx, (unsigned)((rows / 32 + W - 1) / W)),
                           dim3(64 * W), 0, stream, x, ldx, rows, cols, mask, codes, scales, nullptr, nullptr,
                           (uint64_t)0, nullptr, 0, 0, 0, nullptr, nullptr, 0u, panels ? 1 : 0);
    } else {
        constexpr int W = tr_waves<F, false, -1, false>();
        hipLaunchKernelGGL((k_quantize_transpose<F, ROTATE, false>), dim3(tx, (unsigned)((rows / 32 + W - 1) / W)),
                           dim3(64 * W), 0, stream, x, ldx, rows, cols, mask, codes, scales, nullptr, nullptr,
                           (uint64_t)0, nullptr, 0, 0, 0, nullptr, nullptr, 0u, panels ? 1 : 0);
    }
    return hipGetLastError();
}

template <int F, bool ROTATE>
hipError_t launch_tr_sr_fmt(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, uint32_t mask, uint64_t seed,
                            uint8_t *codes, uint8_t *scales, hipStream_t stream) {
    const bool vec = ((uintptr_t)x % 8 == 0) && (ldx % 4 == 0) && ((uintptr_t)codes % 16 == 0);
    constexpr int W = tr_waves<F, true, -1, true>();
    static_assert(W == tr_waves<F, false, -1, true>(), "one grid for both variants");
    const dim3 grid((unsigned)((cols + kTrCols - 1) / kTrCols), (unsigned)((rows / 32 + W - 1) / W));
    if (vec)
        hipLaunchKernelGGL((k_quantize_transpose<F, ROTATE, true, -1, true>), grid, dim3(64 * W), 0, stream,
                           x, ldx, rows, cols, mask, codes, scales, nullptr, nullptr, seed);
    else
        hipLaunchKernelGGL((k_quantize_transpose<F, ROTATE, false, -1, true>), grid, dim3(64 * W), 0, stream,
                           x, ldx, rows, cols, mask, codes, scales, nullptr, nullptr, seed);
    return hipGetLastError();
}

// Both operands of a GEMM in one launch (see mx_quantize_pair): the second
// tensor's workgroups follow the first's.  Tensors that need different
// kernel variants (row strides, alignment) take two launches instead.
template <int F>
hipError_t launch_rows_pair_fmt(const QuantJob &a, const QuantJob &b, hipStream_t stream) {
    const uint32_t per_block = kRowThreads * kRowUnroll;
    auto flags = [](const QuantJob &j, bool &contig, bool &vec) {
        contig = j.ldx == j.cols;
        vec = ((uintptr_t)j.x % 16 == 0) && (j.ldx % 8 == 0) && ((uintptr_t)j.codes % (F == E2M1 ? 4 : 8) == 0);
    };
    bool ca, va, cb, vb;
    flags(a, ca, va);
    flags(b, cb, vb);
    const uint64_t ta = (uint64_t)a.rows * (uint64_t)a.cols / 8, tb = (uint64_t)b.rows * (uint64_t)b.cols / 8;
    const uint64_t ga = (ta + per_block - 1) / per_block, gb = (tb + per_block - 1) / per_block;
    if (!(ca && va && cb && vb) || ga + gb >= ((uint64_t)1 << 31)) {
        const hipError_t e = launch_rows_fmt<F>(a.x, a.rows, a.cols, a.ldx, a.codes, a.scales, stream);
        return e != hipSuccess ? e : launch_rows_fmt<F>(b.x, b.rows, b.cols, b.ldx, b.codes, b.scales, stream);
    }
    const FastDiv da((uint32_t)(a.cols / 8)), db((uint32_t)(b.cols / 8));
    hipLaunchKernelGGL((k_quantize_rows<F, true, true, true>), dim3((unsigned)(ga + gb)), dim3(kRowThreads), 0, stream,
                       a.x, a.ldx, (uint32_t)ta, (uint32_t)(a.cols / 8), da, a.codes, a.scales,
                       b.x, b.ldx, (uint32_t)tb, (uint32_t)(b.cols / 8), db, b.codes, b.scales, (uint32_t)ga);
    return hipGetLastError();
}

template <int F, bool ROTATE>
hipError_t launch_tr_pair_fmt(const QuantJob &a, const QuantJob &b, uint32_t mask, hipStream_t stream,
                              bool panels) {
    auto vec = [](const QuantJob &j) {
        return ((uintptr_t)j.x % 8 == 0) && (j.ldx % 4 == 0) && ((uintptr_t)j.codes % 16 == 0);
    };
    if (!vec(a) || !vec(b)) {
        const hipError_t e =
            launch_tr_fmt<F, ROTATE>(a.x, a.rows, a.cols, a.ldx, mask, a.codes, a.scales, stream, panels);
        return e != hipSuccess
                   ? e
                   : launch_tr_fmt<F, ROTATE>(b.x, b.rows, b.cols, b.ldx, mask, b.codes, b.scales, stream, panels);
    }
    const uint32_t tx = (uint32_t)((a.cols + kTrCols - 1) / kTrCols), ux = (uint32_t)((b.cols + kTrCols - 1) / kTrCols);
    constexpr int W = tr_waves<F, true, -1, false>();
    const int64_t ra = (a.rows / 32 + W - 1) / W, rb = (b.rows / 32 + W - 1) / W;
    const dim3 grid(tx + ux, (unsigned)(ra > rb ? ra : rb));
    hipLaunchKernelGGL((k_quantize_transpose<F, ROTATE, true, -1, false, true>), grid, dim3(64 * W), 0, stream,
                       a.x, a.ldx, a.rows, a.cols, mask, a.codes, a.scales, nullptr, nullptr, (uint64_t)0,
                       b.x, b.ldx, b.rows, b.cols, b.codes, b.scales, tx, panels ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_transpose_sr(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                        bool rotate, uint32_t sign_mask, uint64_t seed, uint8_t *codes,
                                        uint8_t *scales, hipStream_t stream) {
    if (rotate) {
        switch (fmt) {
        case E4M3: return launch_tr_sr_fmt<E4M3, true>(x, rows, cols, ldx, sign_mask, seed, codes, scales, stream);
        case E5M2: return launch_tr_sr_fmt<E5M2, true>(x, rows, cols, ldx, sign_mask, seed, codes, scales, stream);
        default: return launch_tr_sr_fmt<E2M1, true>(x, rows, cols, ldx, sign_mask, seed, codes, scales, stream);
        }
    }
    switch (fmt) {
    case E4M3: return launch_tr_sr_fmt<E4M3, false>(x, rows, cols, ldx, 0, seed, codes, scales, stream);
    case E5M2: return launch_tr_sr_fmt<E5M2, false>(x, rows, cols, ldx, 0, seed, codes, scales, stream);
    default: return launch_tr_sr_fmt<E2M1, false>(x, rows, cols, ldx, 0, seed, codes, scales, stream);
    }
}

hipError_t launch_quantize_rows(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                uint8_t *codes, uint8_t *scales, hipStream_t stream) {
    switch (fmt) {
    case E4M3: return launch_rows_fmt<E4M3>(x, rows, cols, ldx, codes, scales, stream);
    case E5M2: return launch_rows_fmt<E5M2>(x, rows, cols, ldx, codes, scales, stream);
    default: return launch_rows_fmt<E2M1>(x, rows, cols, ldx, codes, scales, stream);
    }
}

hipError_t launch_quantize_rows_strided(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                        uint8_t *codes, int64_t ld_codes, uint8_t *scales, int64_t ld_scales,
                                        hipStream_t stream) {
    switch (fmt) {
    case E4M3: return launch_rows_strided_fmt<E4M3>(x, rows, cols, ldx, codes, ld_codes, scales, ld_scales, stream);
    case E5M2: return launch_rows_strided_fmt<E5M2>(x, rows, cols, ldx, codes, ld_codes, scales, ld_scales, stream);
    default: return launch_rows_strided_fmt<E2M1>(x, rows, cols, ldx, codes, ld_codes, scales, ld_scales, stream);
    }
}

hipError_t launch_quantize_transpose(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx,
                                     int fmt, bool rotate, uint32_t sign_mask, uint8_t *codes,
                                     uint8_t *scales, hipStream_t stream, bool panels) {
    if (rotate) {
        switch (fmt) {
        case E4M3: return launch_tr_fmt<E4M3, true>(x, rows, cols, ldx, sign_mask, codes, scales, stream, panels);
        case E5M2: return launch_tr_fmt<E5M2, true>(x, rows, cols, ldx, sign_mask, codes, scales, stream, panels);
        default: return launch_tr_fmt<E2M1, true>(x, rows, cols, ldx, sign_mask, codes, scales, stream, panels);
        }
    }
    switch (fmt) {
    case E4M3: return launch_tr_fmt<E4M3, false>(x, rows, cols, ldx, 0, codes, scales, stream, panels);
    case E5M2: return launch_tr_fmt<E5M2, false>(x, rows, cols, ldx, 0, codes, scales, stream, panels);
    default: return launch_tr_fmt<E2M1, false>(x, rows, cols, ldx, 0, codes, scales, stream, panels);
    }
}

hipError_t launch_quantize_pair(int mode, int fmt, uint32_t sign_mask, const QuantJob &a, const QuantJob &b,
                                hipStream_t stream) {
    if (mode == 0) {
        switch (fmt) {
        case E4M3: return launch_rows_pair_fmt<E4M3>(a, b, stream);
        case E5M2: return launch_rows_pair_fmt<E5M2>(a, b, stream);
        default: return launch_rows_pair_fmt<E2M1>(a, b, stream);
        }
    }
    const bool panels = mode >= 3;  // 3, 4: modes 1, 2 with K-panel output
    if (mode == 2 || mode == 4) {
        switch (fmt) {
        case E4M3: return launch_tr_pair_fmt<E4M3, true>(a, b, sign_mask, stream, panels);
        case E5M2: return launch_tr_pair_fmt<E5M2, true>(a, b, sign_mask, stream, panels);
        default: return launch_tr_pair_fmt<E2M1, true>(a, b, sign_mask, stream, panels);
        }
    }
    switch (fmt) {
    case E4M3: return launch_tr_pair_fmt<E4M3, false>(a, b, 0, stream, panels);
    case E5M2: return launch_tr_pair_fmt<E5M2, false>(a, b, 0, stream, panels);
    default: return launch_tr_pair_fmt<E2M1, false>(a, b, 0, stream, panels);
    }
}

}  // namespace mx
