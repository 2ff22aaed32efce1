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

MXHD int clz32(uint32_t v) {  // v != 0
#if defined(__HIP_DEVICE_COMPILE__)
    return __clz(v);
#else
    return __builtin_clz(v);
#endif
}

// ---------------------------------------------------------------------------
// Block scale exponent e = clamp(floor(log2 amax) - EMAX, -127, 127).

// amax given as bf16 magnitude bits (bits & 0x7FFF), finite.
template <int F>
MXHD int scale_exp_bf16(uint32_t amax_bits) {
    int fl;
    if (amax_bits >= 0x80u)
        fl = (int)(amax_bits >> 7) - 127;          // normal: exponent field - bias
    else if (amax_bits == 0u)
        return -127;                               // all-zero block
    else
        fl = (31 - clz32(amax_bits)) - 133;        // subnormal: m * 2^-133
    int e = fl - Traits<F>::EMAX;
    e = e < -127 ? -127 : e;
    return e > 127 ? 127 : e;
}

// amax given as fp32 magnitude bits (bits & 0x7FFFFFFF), finite.
template <int F>
MXHD int scale_exp_f32(uint32_t amax_bits) {
    int fl;
    if (amax_bits >= 0x00800000u)
        fl = (int)(amax_bits >> 23) - 127;
    else if (amax_bits == 0u)
        return -127;
    else
        fl = (31 - clz32(amax_bits)) - 149;        // subnormal: m * 2^-149
    int e = fl - Traits<F>::EMAX;
    e = e < -127 ? -127 : e;
    return e > 127 ? 127 : e;
}

}  // namespace mx
