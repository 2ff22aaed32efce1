// mx_convert.h -- E8M0 scale exponents for the MX quantizers (gfx950 path).
//
// MX micro-scaling (FP4-training article on hzrcw.cc, section 02: one dynamic
// exponent per small block; block size 32 per the MindSpeed-LLM FSDP2 page)
// with the OCP element encodings E4M3 (bias 7, max 448, no Inf), E5M2 (bias
// 15, max normal 57344) and E2M1 (bias 1, max 6), and the E8M0 block scale
//     S = clamp(floor(log2 amax) - emax, -127, 127) + 127.
// The element casts themselves are the gfx950 scaled conversion instructions
// (mx_quant_kernels.h).
//
// Everything here is plain integer code usable from host and device, so that
// a CPU build can check it exhaustively.  MXHD expands to __host__ __device__
// under hipcc and to nothing in a plain C++ build.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define MXHD __host__ __device__ __forceinline__
#else
#define MXHD inline
#endif

namespace mx {

enum Fmt : int { E4M3 = 0, E5M2 = 1, E2M1 = 2 };

// EMAX: exponent of the largest normal binade of the element format.
template <int F> struct Traits;
template <> struct Traits<E4M3> { static constexpr int EMAX = 8; };    // 448 = 1.75 * 2^8
template <> struct Traits<E5M2> { static constexpr int EMAX = 15; };   // 57344 = 1.75 * 2^15
template <> struct Traits<E2M1> { static constexpr int EMAX = 2; };    // 6 = 1.5 * 2^2

// ---------------------------------------------------------------------------
// Block scale exponent e = clamp(floor(log2 amax) - EMAX, -127, 127).
//
// For a finite amax this is max(E - bias - EMAX, -127), E the amax's exponent
// field: a normal amax has floor(log2 amax) = E - bias; a subnormal one (E = 0)
// or zero lies below 2^(1 - bias) <= 2^-126, so its exponent reaches the lower
// clamp anyway, as E = 0 gives; and E <= 254 keeps e <= 127 - EMAX, below the
// upper clamp.  No leading-zero count and no branch.

// amax given as bf16 magnitude bits (bits & 0x7FFF), finite.
template <int F>
MXHD int scale_exp_bf16(uint32_t amax_bits) {
    const int e = (int)(amax_bits >> 7) - 127 - Traits<F>::EMAX;
    return e < -127 ? -127 : e;
}

// amax given as fp32 magnitude bits (bits & 0x7FFFFFFF), finite.
template <int F>
MXHD int scale_exp_f32(uint32_t amax_bits) {
    const int e = (int)(amax_bits >> 23) - 127 - Traits<F>::EMAX;
    return e < -127 ? -127 : e;
}

}  // namespace mx
