// mx_convert.h -- element conversion for the MX quantizers (gfx950 path).
//
// MX micro-scaling (FP4-training article on hzrcw.cc, section 02: one dynamic
// exponent per small block; block size 32 per the MindSpeed-LLM FSDP2 page)
// with the OCP element encodings E4M3 (bias 7, max 448, no Inf), E5M2 (bias
// 15, max normal 57344) and E2M1 (bias 1, max 6), and the E8M0 block scale
//     S = clamp(floor(log2 amax) - emax, -127, 127) + 127.
// Elements are v * 2^-(S-127), rounded to nearest with ties to even and
// saturated to the largest normal; the sign of zero is kept.
//
// Everything here is plain integer / fp32 code usable from host and device,
// so that a CPU build can check it exhaustively.  MXHD expands to
// __host__ __device__ under hipcc and to nothing in a plain C++ build.
#pragma once
#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define MXHD __host__ __device__ __forceinline__
#else
#include <math.h>
#define MXHD inline
#endif

namespace mx {

enum Fmt : int { E4M3 = 0, E5M2 = 1, E2M1 = 2 };

// M: mantissa bits, BIAS, EMIN: exponent of the smallest normal binade,
// EMAX: exponent of the largest normal binade, MAXCODE: code of +max normal,
// SIGN: position of the sign bit in the code.
template <int F> struct Traits;
template <> struct Traits<E4M3> {
    static constexpr int M = 3, BIAS = 7, EMIN = -6, EMAX = 8, MAXCODE = 0x7E, SIGN = 7;
};
template <> struct Traits<E5M2> {
    static constexpr int M = 2, BIAS = 15, EMIN = -14, EMAX = 15, MAXCODE = 0x7B, SIGN = 7;
};
template <> struct Traits<E2M1> {
    static constexpr int M = 1, BIAS = 1, EMIN = 0, EMAX = 2, MAXCODE = 0x7, SIGN = 3;
};

MXHD uint32_t f2u(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __float_as_uint(f);
#else
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
#endif
}

MXHD float u2f(uint32_t u) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __uint_as_float(u);
#else
    float f;
    memcpy(&f, &u, 4);
    return f;
#endif
}

MXHD int clz32(uint32_t v) {  // v != 0
#if defined(__HIP_DEVICE_COMPILE__)
    return __clz(v);
#else
    return __builtin_clz(v);
#endif
}

MXHD float ldexp_f32(float x, int n) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_ldexpf(x, n);
#else
    return ldexpf(x, n);
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

// ---------------------------------------------------------------------------
// Element code of a bf16 value b (16-bit pattern) in a block with scale
// exponent e (amax finite).
//
// The value is moved with ldexp to t = |v| * 2^(-e - 126 - EMIN): the target
// format's smallest normal 2^EMIN lands on fp32's smallest normal 2^-126, and
// since EMIN + BIAS = 1 the fp32 exponent field of t equals the target's
// biased exponent.  Target subnormals become fp32 subnormals, whose bit
// patterns are uniformly spaced, so one integer round-to-nearest-even of the
// fp32 pattern by 23 - M bits yields the code for every binade, carries into
// the next binade included.  ldexp rounds only when t is an fp32 subnormal
// with bits below 2^-149; a bf16 value has 8 significant bits, so that
// happens only for t < 2^-142, far below the first rounding threshold
// 2^(-127 - M), where the code is 0 either way.  The exponent shift is split
// in two ldexp steps so that neither factor leaves the fp32 range.
template <int F>
MXHD uint32_t code_from_bf16(uint32_t b, int e) {
    using T = Traits<F>;
    constexpr int SH = 23 - T::M;
    float v = u2f((b & 0x7FFFu) << 16);                // |v| as fp32, exact
    float t = ldexp_f32(ldexp_f32(v, -e), -126 - T::EMIN);
    uint32_t u = f2u(t);
    uint32_t r = (u + ((1u << (SH - 1)) - 1u) + ((u >> SH) & 1u)) >> SH;
    r = r < (uint32_t)T::MAXCODE ? r : (uint32_t)T::MAXCODE;
    return r | (((b >> 15) & 1u) << T::SIGN);
}

// Element code of an fp32 value y (any finite fp32) in a block with scale
// exponent e.  q = |y| * 2^-e is exact whenever q >= 2^-126; smaller q round
// to code 0 in every format.  Normal targets (q >= 2^EMIN) round the fp32
// pattern of q by 23 - M bits and rebias; subnormal targets add the constant
// 2^(EMIN - M + 23), whose fp32 spacing is the target's subnormal spacing,
// so the hardware add performs the one round-to-nearest-even step.
template <int F>
MXHD uint32_t code_from_f32(float y, int e) {
    using T = Traits<F>;
    constexpr int SH = 23 - T::M;
    const uint32_t yb = f2u(y);
    const float q = ldexp_f32(u2f(yb & 0x7FFFFFFFu), -e);
    const uint32_t u = f2u(q);
    // normal: ((u + half - 1 + lsb) >> SH) - ((127 - BIAS) << M), the rebias
    // folded in before the shift (u >= (127 - BIAS) << 23 holds here)
    const uint32_t rn = (u + ((1u << (SH - 1)) - 1u) - ((uint32_t)(127 - T::BIAS) << 23) +
                         ((u >> SH) & 1u)) >> SH;
    const float magic = u2f((uint32_t)(127 + T::EMIN - T::M + 23) << 23);
    const uint32_t rs = f2u(q + magic) - f2u(magic);
    uint32_t r = (u >= ((uint32_t)(127 + T::EMIN) << 23)) ? rn : rs;
    r = r < (uint32_t)T::MAXCODE ? r : (uint32_t)T::MAXCODE;
    return r | ((yb >> 31) << T::SIGN);
}

}  // namespace mx
