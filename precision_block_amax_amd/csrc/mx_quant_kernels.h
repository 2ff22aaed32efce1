// mx_quant_kernels.h -- the MX quantizer kernels for gfx950 (row mode,
// transposed mode, transposed mode after the fixed-sign 32-point block
// rotation, and the fused form that writes the row and the transposed form
// from one read), shared by the launchers in mx_quant.hip and
// mx_quant_dual.hip.  The design notes are at the top of mx_quant.hip.
#pragma once
#include "mx_internal.h"


namespace mx {
namespace {

constexpr uint32_t kRowThreads = 256;
// 16-byte loads per lane.  Two, read non-temporally (x is streamed once):
// 76% of 8 TB/s on the 28672 x 4096 weight against 71-73% with four, the
// same on the 64 MiB activations (62-65%, a plain copy's rate at that size).
constexpr uint32_t kRowUnroll = 2;

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// max over the four lanes of a DPP quad (lanes 4q .. 4q+3)
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));  // lane ^ 1
    v = umax(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));  // lane ^ 2
    return v;
}

// ---------------------------------------------------------------------------
// Element casts by the gfx950 scaled conversions (v_cvt_scalef32_pk_*): they
// convert v / scale, scale = 2^e, rounding to nearest with ties to even and
// keeping the sign of zero.  E2M1 saturates to +-6, which is exactly the
// saturating MX cast.  E4M3 and E5M2 would round inputs just below the
// saturation point up to the NaN / Inf code, so those values are first
// clamped to +-max_normal * 2^e (one med3), after which they equal the
// saturating cast too.  Both facts were measured on the device against a
// software cast (every bf16 input at every reachable scale exponent, every
// fp32 input at e = 0 and strided fp32 sweeps at nine exponents from -127 to
// 125, zero mismatches); the parity tests run every finite bf16 value at every
// reachable scale through both quantizers.  Element 2k goes to the low
// nibble / byte.
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

template <int F> struct MaxNormal;
template <> struct MaxNormal<E4M3> { static constexpr float v = 448.0f; };
template <> struct MaxNormal<E5M2> { static constexpr float v = 57344.0f; };

// four FP8 codes of a..d (fp32) -> bytes 0..3
template <int F>
__device__ __forceinline__ uint32_t cvt4_fp8(float a, float b, float c, float d, float s, float lim) {
    a = __builtin_amdgcn_fmed3f(a, -lim, lim);
    b = __builtin_amdgcn_fmed3f(b, -lim, lim);
    c = __builtin_amdgcn_fmed3f(c, -lim, lim);
    d = __builtin_amdgcn_fmed3f(d, -lim, lim);
    v2s w = {0, 0};
    if constexpr (F == E4M3) {
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, s, false);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, s, true);
    } else {
        w = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(w, a, b, s, false);
        w = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(w, c, d, s, true);
    }
    return __builtin_bit_cast(uint32_t, w);
}

// eight E2M1 codes of y[0..7] (fp32) -> nibbles 0..7
__device__ __forceinline__ uint32_t cvt8_fp4(const float *y, float s) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], s, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], s, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], s, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], s, 3);
    return w;
}

// eight E2M1 codes of the bf16 pairs d[0..3] (element 2k in the low half of d[k])
__device__ __forceinline__ uint32_t cvt8_fp4_bf16(const uint32_t *d, float s) {
    uint32_t w = 0;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf, d[0]), s, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf, d[1]), s, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf, d[2]), s, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(v2bf, d[3]), s, 3);
    return w;
}

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// ---------------------------------------------------------------------------
// Row mode.  Octet o covers elements 8o .. 8o+7 of the row-major [rows x cols]
// view; cols % 32 == 0 keeps every block inside one quad of lanes.  With
// PAIR, workgroups from `split` on quantize a second tensor (x1 ...), so that
// both operands of a GEMM take one launch.  With OSTR, row r's codes start at
// codes + r * ldco and its scales at scales + r * ldsc (bytes), e.g. rows of
// [codes | scales] in one buffer.
template <int F, bool CONTIG, bool VEC, bool PAIR = false, bool OSTR = false>
__global__ __launch_bounds__(kRowThreads) void k_quantize_rows(
    const uint16_t *__restrict__ x, int64_t ldx, uint32_t total_oct, uint32_t oct_per_row,
    FastDiv row_div, uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
    const uint16_t *__restrict__ x1 = nullptr, int64_t ldx1 = 0, uint32_t total_oct1 = 0,
    uint32_t oct_per_row1 = 0, FastDiv row_div1 = FastDiv(), uint8_t *__restrict__ codes1 = nullptr,
    uint8_t *__restrict__ scales1 = nullptr, uint32_t split = 0, int64_t ldco = 0, int64_t ldsc = 0) {
    uint32_t blk = blockIdx.x;
    if (PAIR && blk >= split) {  // uniform across the workgroup
        blk -= split;
        x = x1; ldx = ldx1; total_oct = total_oct1; oct_per_row = oct_per_row1; row_div = row_div1;
        codes = codes1; scales = scales1;
    }
    const uint32_t o0 = blk * (kRowThreads * kRowUnroll) + threadIdx.x;
    uint32_t w[kRowUnroll][4];

#pragma unroll
    for (uint32_t u = 0; u < kRowUnroll; u++) {
        const uint32_t o = o0 + u * kRowThreads;
        w[u][0] = w[u][1] = w[u][2] = w[u][3] = 0;
        if (o < total_oct) {
            const uint16_t *p;
            if (CONTIG) {
                p = x + (uint64_t)o * 8;
            } else {
                const uint32_t r = row_div.div(o);
                p = x + (int64_t)r * ldx + (uint64_t)(o - r * oct_per_row) * 8;
            }
            if (VEC) {
                typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
                w[u][0] = t[0]; w[u][1] = t[1]; w[u][2] = t[2]; w[u][3] = t[3];
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++) w[u][i] = (uint32_t)p[2 * i] | ((uint32_t)p[2 * i + 1] << 16);
            }
        }
    }

#pragma unroll
    for (uint32_t u = 0; u < kRowUnroll; u++) {
        const uint32_t o = o0 + u * kRowThreads;
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t a = w[u][i] & 0x7FFF7FFFu;
            m = umax(m, umax(a & 0xFFFFu, a >> 16));
        }
        m = quad_max(m);  // every lane runs the exchange; out-of-range quads hold zeros
        const bool finite = m < 0x7F80u;
        const int e = scale_exp_bf16<F>(finite ? m : 0u);
        const float sc = __builtin_amdgcn_ldexpf(1.0f, e);
        uint32_t packed = 0, lo = 0, hi = 0;
        if constexpr (F == E2M1) {
            packed = finite ? cvt8_fp4_bf16(w[u], sc) : 0u;
        } else {
            const float lim = __builtin_amdgcn_ldexpf(MaxNormal<F>::v, e);
            lo = cvt4_fp8<F>(bf16_lo(w[u][0]), bf16_hi(w[u][0]), bf16_lo(w[u][1]), bf16_hi(w[u][1]), sc, lim);
            hi = cvt4_fp8<F>(bf16_lo(w[u][2]), bf16_hi(w[u][2]), bf16_lo(w[u][3]), bf16_hi(w[u][3]), sc, lim);
            lo = finite ? lo : 0u;
            hi = finite ? hi : 0u;
        }
        if (o < total_oct) {
            constexpr int CB = F == E2M1 ? 4 : 8;  // code bytes per octet
            uint8_t *cp, *sp;
            if (OSTR) {
                const uint32_t r = row_div.div(o), c = o - r * oct_per_row;
                cp = codes + (int64_t)r * ldco + (uint64_t)c * CB;
                sp = scales + (int64_t)r * ldsc + (c >> 2);
            } else {
                cp = codes + (uint64_t)o * CB;
                sp = scales + (o >> 2);
            }
            if (F == E2M1) {
                if (VEC) {
                    *reinterpret_cast<uint32_t *>(cp) = packed;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++) cp[i] = (uint8_t)(packed >> (8 * i));
                }
            } else {
                if (VEC) {
                    *reinterpret_cast<uint2 *>(cp) = make_uint2(lo, hi);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        cp[i] = (uint8_t)(lo >> (8 * i));
                        cp[4 + i] = (uint8_t)(hi >> (8 * i));
                    }
                }
            }
            if ((threadIdx.x & 3u) == 0) *sp = (uint8_t)(finite ? e + 127 : 0xFF);
        }
    }
}

// ---------------------------------------------------------------------------
// Transposed mode, optionally after the rotation.  Lane: 4 columns
// c0 .. c0+3 of one 32-row block at a time (one 8-byte load per row, each
// wave instruction reading 512 contiguous bytes of a row), so the block's
// amax and the rotation's butterflies stay in the lane's registers.  A
// workgroup covers 256 columns x W row blocks, one block per wave (W below).
// The codes are staged in LDS and written out afterwards as whole runs of W
// blocks of each output row (128 bytes for E2M1, 512 for FP8 with W = 16),
// and the W scale bytes of each output row as one store.
constexpr int kTrColsPerLane = 4;
constexpr int kTrCols = 256;   // columns per workgroup
// Waves per workgroup, one row block each.  FP8 codes alone: 16, so each
// output row leaves as a 512-byte run (measured 8% faster than 8 waves with
// 256-byte runs on the 8192 x 8192 weight).  E2M1 (128-byte runs), the fused
// row form, stochastic rounding and unaligned inputs: 8 (16 waves measured
// 10-15% slower for E2M1; the others do not fit 16 waves' registers or LDS).
template <int F, bool VEC, int FR, bool SR>
constexpr int tr_waves() { return (F != E2M1 && VEC && FR < 0 && !SR) ? 16 : 8; }

// y = c * H32 * diag(s) * x, stages h = 1, 2, 4, 8, 16, one fp32 rounding per op
__device__ __forceinline__ void hadamard32(float (&y)[32], uint32_t sign_mask) {
    if (sign_mask) {
#pragma unroll
        for (int i = 0; i < 32; i++) y[i] = __uint_as_float(__float_as_uint(y[i]) ^ (((sign_mask >> i) & 1u) << 31));
    }
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 32; j++) {
            if (!(j & h)) {
                const float a = y[j], b = y[j + h];
                y[j] = __fadd_rn(a, b);
                y[j + h] = __fsub_rn(a, b);
            }
        }
    }
    const float c = __uint_as_float(0x3E3504F3u);  // RN_fp32(1/sqrt(32))
#pragma unroll
    for (int i = 0; i < 32; i++) y[i] = __fmul_rn(y[i], c);
}

// ---------------------------------------------------------------------------
// Stochastic rounding (the randomised cast the FP4-training article, section
// 01, names as the common alternative to its deterministic scheme).  The rule:
// with lo <= |q| < hi the neighbouring grid magnitudes, round up iff the
// element's 32-bit random word r < floor(2^32 (|q| - lo) / (hi - lo));
// saturate at the largest normal; keep the sign.  Random words come from
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): element i of the output takes word i mod 4 of the
// block at counter (i / 4, 0, 0) under key (seed low, seed high).
struct U4 { uint32_t x, y, z, w; };
__device__ __forceinline__ U4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1) {
    uint32_t c2 = 0, c3 = 0;
#pragma unroll
    for (int round = 0; round < 10; round++) {
        // multipliers and key increments of the published generator
        const uint32_t h0 = __umulhi(0xD2511F53u, c0), l0 = 0xD2511F53u * c0;
        const uint32_t h1 = __umulhi(0xCD9E8D57u, c2), l1 = 0xCD9E8D57u * c2;
        const uint32_t n0 = h1 ^ c1 ^ k0, n2 = h0 ^ c3 ^ k1;
        c0 = n0; c1 = l1; c2 = n2; c3 = l0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return U4{c0, c1, c2, c3};
}

// Grid parameters of the element formats: mantissa bits, exponent of the
// smallest normal binade, largest normal.
template <int F> struct Grid;
template <> struct Grid<E4M3> { static constexpr int M = 3, EMIN = -6; static constexpr float MAX = 448.0f; };
template <> struct Grid<E5M2> { static constexpr int M = 2, EMIN = -14; static constexpr float MAX = 57344.0f; };
template <> struct Grid<E2M1> { static constexpr int M = 1, EMIN = 0; static constexpr float MAX = 6.0f; };

// the grid value (unscaled, signed) that y * 2^-e rounds to under word r.
// q = y * 2^-e is exact wherever it is an fp32 normal; below that every
// format's spacing is so much larger that the up-probability truncates to 0
// either way.  t = |q| / spacing, its integer and fractional parts and the
// 32-bit fixed-point fraction are all exact in fp32.
template <int F>
__device__ __forceinline__ float sr_round(float y, int e, uint32_t r) {
    const float q = __builtin_amdgcn_ldexpf(y, -e);
    const float a = __builtin_fabsf(q);
    float mag = Grid<F>::MAX;
    if (a < Grid<F>::MAX) {
        const int k = (int)(__float_as_uint(a) >> 23) - 127;   // -127 for zero and subnormals
        const int kk = k < Grid<F>::EMIN ? Grid<F>::EMIN : k;  // binade whose spacing applies
        const float t = __builtin_amdgcn_ldexpf(a, Grid<F>::M - kk);
        float n = __builtin_floorf(t);
        const uint32_t frac = (uint32_t)__builtin_amdgcn_ldexpf(t - n, 32);  // truncating conversion
        n += r < frac ? 1.0f : 0.0f;
        mag = __builtin_fminf(__builtin_amdgcn_ldexpf(n, kk - Grid<F>::M), Grid<F>::MAX);
    }
    return __builtin_copysignf(mag, q);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// FR >= 0 adds the row form in format FR (the fused dual-direction
// quantizer): row r's block b is x[r, 32b .. 32b+31], i.e. the 4 columns of
// this lane and of the 7 neighbouring lanes 8g .. 8g+7 (cols % 32 == 0, so
// such a group of lanes is either wholly inside the matrix or wholly
// outside).  Its amax is reduced over the group with DPP and each lane
// casts its own 4 elements.  The wave's 32 rows of codes (128 or 256 bytes
// each) and scales (8 bytes each) are collected in the wave's own LDS area
// and written with 16-byte lanes: 4 or 8 store instructions per block
// instead of 32 narrow ones, and one for the scales.
//
// SR selects stochastic rounding of the transposed form (no row form) with
// the random words of `seed`; output element t of output row c is element
// c * rows + t of the generator's stream.
//
// PAIR: workgroup columns from `split` on quantize a second tensor (x1 ...),
// so that both operands of a GEMM take one launch; the grid's rows cover the
// taller of the two, and a workgroup past its tensor's last row block writes
// nothing.
//
// panels != 0 writes the transposed codes K-panel-major: the codes of output
// row c that cover bytes [128 p, 128 p + 128) of the row (K elements
// [256 p, 256 p + 256) for E2M1, [128 p, 128 p + 128) for FP8) sit at
// codes + p * (cols * 128) + c * 128.  A workgroup's output then is whole
// 32 KiB runs instead of 256 runs of 128 or 512 bytes (the GEMM reads either
// layout; the launcher needs rows to be a whole number of panels).  With the
// row form (FR >= 0) its codes go K-panel-major too: bytes [128 p, 128 p + 128)
// of row r at codes_r + p * (rows * 128) + r * 128, so a wave's 32 rows are
// one 4 KiB run per panel (cols a whole number of panels).
template <int F, bool ROTATE, bool VEC, int FR = -1, bool SR = false, bool PAIR = false>
__global__ __launch_bounds__((64 * tr_waves<F, VEC, FR, SR>())) void k_quantize_transpose(
    const uint16_t *__restrict__ x, int64_t ldx, int64_t rows, int64_t cols, uint32_t sign_mask,
    uint8_t *__restrict__ codes, uint8_t *__restrict__ scales, uint8_t *__restrict__ codes_r = nullptr,
    uint8_t *__restrict__ scales_r = nullptr, uint64_t seed = 0, const uint16_t *__restrict__ x1 = nullptr,
    int64_t ldx1 = 0, int64_t rows1 = 0, int64_t cols1 = 0, uint8_t *__restrict__ codes1 = nullptr,
    uint8_t *__restrict__ scales1 = nullptr, uint32_t split = 0, int panels = 0) {
    static_assert(!(SR && FR >= 0), "stochastic rounding is a transposed-form variant");
    static_assert(!(PAIR && (SR || FR >= 0)), "pairs of the plain and rotated transposed forms only");
    constexpr int kTrWaves = tr_waves<F, VEC, FR, SR>(), kTrBlocks = kTrWaves;
    uint32_t bx = blockIdx.x;
    if (PAIR && bx >= split) {  // uniform across the workgroup
        bx -= split;
        x = x1; ldx = ldx1; rows = rows1; cols = cols1; codes = codes1; scales = scales1;
    }
    constexpr int BB = F == E2M1 ? 16 : 32;             // code bytes per block of one output row
    constexpr int CB = kTrBlocks * BB;                  // staged bytes per output row: 128 or 256
    constexpr int NCH = CB / 16;                        // 16-byte chunks per output row
    __shared__ __attribute__((aligned(16))) uint8_t sC[kTrCols * CB];
    __shared__ __attribute__((aligned(16))) uint8_t sS[kTrCols * kTrBlocks];
    // row form: per wave 32 rows x RB code bytes, then 32 rows x 8 scale bytes
    constexpr int RB = FR == E2M1 ? 128 : 256;
    constexpr int RSTAGE = FR >= 0 ? kTrWaves * 32 * (RB + 8) : 16;
    __shared__ __attribute__((aligned(16))) uint8_t sR[RSTAGE];
    // chunk q of output row c sits at c * CB + ((q ^ key(c)) << 4): the 16
    // lanes of one LDS write pass hold columns 4L + j, whose keys differ
    const auto key = [](int c) { return (c >> 2) & (NCH - 1); };

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t ctile = (int64_t)bx * kTrCols;
    const int64_t rb0 = (int64_t)blockIdx.y * kTrBlocks;
    const int64_t nrb = rows / 32;
    const int nb = (int)((nrb - rb0) < kTrBlocks ? (nrb - rb0) : kTrBlocks);    // valid blocks
    const int nc = (int)((cols - ctile) < kTrCols ? (cols - ctile) : kTrCols);  // valid columns
    const int cl = lane * kTrColsPerLane;                                        // lane's first column in the tile
    const int ncols = nc - cl < kTrColsPerLane ? (nc - cl < 0 ? 0 : nc - cl) : kTrColsPerLane;

    static_assert(kTrWaves == kTrBlocks, "one block per wave");
    const int b = wave;  // block within the workgroup
    if (b < nb && ncols > 0) {  // the barrier below is reached by every wave
        const int64_t rb = rb0 + b;
        // w[i][0] = columns c0, c0+1 of row 32 rb + i; w[i][1] = columns c0+2, c0+3
        uint32_t w[32][2];
        const uint16_t *p = x + rb * 32 * ldx + ctile + cl;
        if (VEC && ncols == kTrColsPerLane) {
            // non-temporal: every input byte is read once (the rotated pair of the weight
            // gradient's operands measured 6% faster than with plain loads)
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int i = 0; i < 32; i++) {
                const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p + i * ldx));
                w[i][0] = t.x;
                w[i][1] = t.y;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 32; i++) {
                uint32_t v[4];
#pragma unroll
                for (int j = 0; j < 4; j++) v[j] = j < ncols ? p[i * ldx + j] : 0u;
                w[i][0] = v[0] | (v[1] << 16);
                w[i][1] = v[2] | (v[3] << 16);
            }
        }
        if constexpr (FR >= 0) {
            const int64_t rcb = FR == E2M1 ? cols / 2 : cols;  // row-form code bytes per row
            const int64_t nsr = cols / 32;                     // row-form scales per row
            uint8_t *rc = sR + wave * 32 * (RB + 8);           // this wave's rows of codes ...
            uint8_t *rs = rc + 32 * RB;                        // ... and of scales
#pragma unroll
            for (int i = 0; i < 32; i += 2) {
                // |bf16| maxima over the lane's 4 columns of rows i (low half) and i + 1 (high half)
                const uint32_t ra = pk_max_u16(w[i][0] & 0x7FFF7FFFu, w[i][1] & 0x7FFF7FFFu);
                const uint32_t rb2 = pk_max_u16(w[i + 1][0] & 0x7FFF7FFFu, w[i + 1][1] & 0x7FFF7FFFu);
                uint32_t m = pk_max_u16(__builtin_amdgcn_perm(rb2, ra, 0x05040100u),
                                        __builtin_amdgcn_perm(rb2, ra, 0x07060302u));
                // over the 8 lanes of the group: swap pairs, swap pairs of pairs, mirror halves of 8
                m = pk_max_u16(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));
                m = pk_max_u16(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));
                m = pk_max_u16(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x141, 0xF, 0xF, false));
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int r = i + h;
                    const uint32_t mr = h ? (m >> 16) : (m & 0xFFFFu);
                    const bool fin = mr < 0x7F80u;
                    const int er = scale_exp_bf16<FR>(fin ? mr : 0u);
                    const float sr = __builtin_amdgcn_ldexpf(1.0f, er);
                    if constexpr (FR == E2M1) {
                        uint32_t q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(0u, __builtin_bit_cast(v2bf, w[r][0]), sr, 0);
                        q = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(q, __builtin_bit_cast(v2bf, w[r][1]), sr, 1);
                        *reinterpret_cast<uint16_t *>(&rc[r * RB + 2 * lane]) = (uint16_t)(fin ? q : 0u);
                    } else {
                        const float lim = __builtin_amdgcn_ldexpf(MaxNormal<FR>::v, er);
                        const uint32_t q = cvt4_fp8<FR>(bf16_lo(w[r][0]), bf16_hi(w[r][0]), bf16_lo(w[r][1]),
                                                        bf16_hi(w[r][1]), sr, lim);
                        *reinterpret_cast<uint32_t *>(&rc[r * RB + 4 * lane]) = fin ? q : 0u;
                    }
                    if ((lane & 7) == 0) rs[r * 8 + (lane >> 3)] = (uint8_t)(fin ? er + 127 : 0xFF);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kTrColsPerLane; j++) {
            if (j >= ncols) break;
            float y[32];
#pragma unroll
            for (int i = 0; i < 32; i++) y[i] = (j & 1) ? bf16_hi(w[i][j >> 1]) : bf16_lo(w[i][j >> 1]);
            if (ROTATE) hadamard32(y, sign_mask);
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < 32; i++) m = umax(m, __float_as_uint(y[i]) & 0x7FFFFFFFu);
            // bf16 inputs are exact in fp32, so the fp32 scale rule gives the bf16 one
            const bool finite = m < 0x7F800000u;
            const int e = scale_exp_f32<F>(finite ? m : 0u);
            float sc = __builtin_amdgcn_ldexpf(1.0f, e);
            const int c = cl + j;
            if constexpr (SR) {
                // replace y by its stochastically rounded grid values; the casts below then see
                // representable values at scale 1 and are exact
                const uint64_t base = ((uint64_t)(ctile + c) * (uint64_t)rows + (uint64_t)(rb * 32)) >> 2;
                const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
                for (int g = 0; g < 8; g++) {
                    const uint64_t ctr = base + g;
                    const U4 r = philox4x32_10((uint32_t)ctr, (uint32_t)(ctr >> 32), k0, k1);
                    y[4 * g + 0] = sr_round<F>(y[4 * g + 0], e, r.x);
                    y[4 * g + 1] = sr_round<F>(y[4 * g + 1], e, r.y);
                    y[4 * g + 2] = sr_round<F>(y[4 * g + 2], e, r.z);
                    y[4 * g + 3] = sr_round<F>(y[4 * g + 3], e, r.w);
                }
                sc = 1.0f;
            }
            if constexpr (F == E2M1) {
                uint32_t q[4];
#pragma unroll
                for (int k = 0; k < 4; k++) q[k] = finite ? cvt8_fp4(y + 8 * k, sc) : 0u;
                *reinterpret_cast<uint4 *>(&sC[c * CB + ((b ^ key(c)) << 4)]) = make_uint4(q[0], q[1], q[2], q[3]);
            } else {
                const float lim = SR ? MaxNormal<F>::v : __builtin_amdgcn_ldexpf(MaxNormal<F>::v, e);
                uint32_t q[8];
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const uint32_t v = cvt4_fp8<F>(y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3], sc, lim);
                    q[k] = finite ? v : 0u;
                }
                *reinterpret_cast<uint4 *>(&sC[c * CB + (((2 * b) ^ key(c)) << 4)]) = make_uint4(q[0], q[1], q[2], q[3]);
                *reinterpret_cast<uint4 *>(&sC[c * CB + (((2 * b + 1) ^ key(c)) << 4)]) = make_uint4(q[4], q[5], q[6], q[7]);
            }
            sS[c * kTrBlocks + b] = (uint8_t)(finite ? e + 127 : 0xFF);
        }
    }
    if constexpr (FR >= 0) {
        if (b < nb) {  // wave-uniform: every lane of the wave takes part in the write-out
            const int64_t rcb = FR == E2M1 ? cols / 2 : cols;
            const int64_t nsr = cols / 32;
            const int64_t rb = rb0 + b;
            const uint8_t *rc = sR + wave * 32 * (RB + 8);
            const uint8_t *rs = rc + 32 * RB;
            // write-out of the wave's rows (LDS operations of one wave complete in order, so the
            // reads below see every lane's writes above): lane t copies 16-byte chunk t % (RB / 16)
            // of row t / (RB / 16), skipping chunks past the last column
            constexpr int CPRr = RB / 16;
            const int vcr = (nc * RB / kTrCols) / 16;        // valid chunks per row
#pragma unroll
            for (int k = 0; k < 32 * CPRr / 64; k++) {
                const int t = k * 64 + lane, r = t / CPRr, q = t % CPRr;
                if (q >= vcr) continue;
                const uint4 v = *reinterpret_cast<const uint4 *>(&rc[r * RB + 16 * q]);
                const int64_t pos = ctile * RB / kTrCols + 16 * q;  // byte of row rb * 32 + r
                uint8_t *dst = panels ? codes_r + (pos >> 7) * (rows * 128) + (rb * 32 + r) * 128 + (pos & 127)
                                      : codes_r + (rb * 32 + r) * rcb + pos;
                if (VEC) {
                    *reinterpret_cast<uint4 *>(dst) = v;
                } else {
                    const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int i = 0; i < 16; i++) dst[i] = (uint8_t)(vv[i >> 2] >> (8 * (i & 3)));
                }
            }
            if (lane < 32) {                                  // one row's 8 (or fewer) scale bytes per lane
                const int vs = nc / 32;
                uint8_t *dst = scales_r + (rb * 32 + lane) * nsr + ctile / 32;
                if (vs == kTrBlocks && ((uintptr_t)dst & 7) == 0) {
                    *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(&rs[lane * 8]);
                } else {
                    for (int i = 0; i < vs; i++) dst[i] = rs[lane * 8 + i];
                }
            }
        }
    }
    __syncthreads();

    // write-out: thread t copies chunk t % NCH of output row t / NCH (+ 256 / NCH per step)
    const int64_t row_bytes = (F == E2M1) ? rows / 2 : rows;
    const int vchunks = nb * BB / 16;                   // valid chunks per output row
#pragma unroll
    for (int k = 0; k < kTrCols * NCH / (64 * kTrWaves); k++) {
        const int t = k * 64 * kTrWaves + threadIdx.x;
        const int c = t / NCH, q = t % NCH;
        if (c >= nc || q >= vchunks) continue;
        const uint4 v = *reinterpret_cast<const uint4 *>(&sC[c * CB + ((q ^ key(c)) << 4)]);
        const int64_t pos = rb0 * BB + q * 16;  // byte of output row ctile + c
        uint8_t *dst = panels ? codes + (pos >> 7) * (cols * 128) + (ctile + c) * 128 + (pos & 127)
                              : codes + (ctile + c) * row_bytes + pos;
        if (VEC) {
            *reinterpret_cast<uint4 *>(dst) = v;
        } else {
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 16; i++) dst[i] = (uint8_t)(vv[i >> 2] >> (8 * (i & 3)));
        }
    }
    {
        const int c = threadIdx.x;  // one output row's 8 scale bytes per thread
        if (c < nc) {
            uint8_t *dst = scales + (ctile + c) * nrb + rb0;
            if (kTrBlocks == 16 && nb == kTrBlocks && (((uintptr_t)dst & 15) == 0)) {
                *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(&sS[c * kTrBlocks]);
            } else if (kTrBlocks == 8 && nb == kTrBlocks && (((uintptr_t)dst & 7) == 0)) {
                *reinterpret_cast<uint2 *>(dst) = *reinterpret_cast<const uint2 *>(&sS[c * kTrBlocks]);
            } else {
                for (int i = 0; i < nb; i++) dst[i] = sS[c * kTrBlocks + i];
            }
        }
    }
}

}  // namespace
}  // namespace mx
