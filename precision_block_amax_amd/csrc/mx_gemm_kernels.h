// mx_gemm_kernels.h -- MX-scaled GEMM kernels for gfx950: C[m, n] = sum_k A[m, k] * B[n, k],
// both operands MX-quantized with K contiguous (codes + one E8M0 scale per
// 32-element block), fp32 accumulation, fp32 or bf16 output.
//
// The linear-layer GEMMs (forward, activation gradient, weight gradient) of
// quantized training (FP4-training article on hzrcw.cc, section 02), which
// the Primus page identifies as the dominant training cost.
//
// The main path is the pipelined kernel at the end of this file (namespace
// pipe): 8 waves of 128 x 64, stage loads straight to LDS, used whenever K is
// a multiple of 512 and the operands are aligned.  The general kernels below
// cover every other shape; they share one tiling (MFMA-bound; 2*M*N*K flops):
//   - workgroup tile 256 x 256, four waves of 128 x 128 (4 x 4 tiles of
//     32 x 32, 256 fp32 accumulators per lane);
//   - operand codes and scales double-buffered in LDS, the 16-byte chunks of
//     each code row XOR-swizzled by the row index so that the lanes reading
//     one K chunk of consecutive rows hit distinct banks; one barrier per K
//     tile, the next tile's global loads in flight during the current tile's
//     matrix work;
//   - workgroups are dealt round-robin to the 8 XCDs, so each XCD gets a
//     contiguous run of tiles, ordered in groups of 8 tile rows, to keep shared
//     A rows and B columns in that XCD's L2;
//   - M and N tails: loads clamp to the last valid row, stores are masked; the
//     K tail is zero-filled (code 0, scale byte 0).
//
// k_gemm_fp4 (E2M1 x E2M1): V_MFMA_SCALE_F32_32X32X64_F8F6F4.  Lane l serves
// row l % 32 of A (column of B); its half h = l / 32 holds K[32h, 32h+32) of
// the 64-element step -- one whole MX block -- and supplies that block's
// E8M0 byte; the matrix core applies both scales.  Measured on gfx950: the
// products of two E2M1 values span few enough binades that the instruction's
// internal sum is exact, so only the fp32 accumulation rounds.
//
// k_gemm_carrier (any pair with an FP8 operand): measured on gfx950, the
// scaled instruction sums the products of an FP8 block in a fixed-point
// window about 13 bits below the largest product (1 + 2^-13 survives, 1 +
// 2^-14 does not), an error of up to ~1e-4 of sum |a*b| on random codes --
// outside the fp32 accumulation tolerance this library is held to.  So FP8
// codes travel as bf16 (every E4M3 / E5M2 / E2M1 value times a power of two
// in [2^-40, 1] is an exact bf16) through V_MFMA_F32_32X32X16_BF16, whose
// 16-product sum is exact with one fp32 rounding:
//   a'[m, k] = code * 2^(S_a[m, b] - R_a[m]),  R_a[m] = max_b S_a[m, b]
// (V_CVT_SCALEF32_PK_BF16_{FP8,BF8,FP4}: two codes per instruction, exact for
// normal power-of-two scales), same for B, and C = 2^(R_a + R_b - 254) *
// sum a' b'.  A tile in which some row's scales spread over more than 40
// binades (the pipelined kernel leaves all-zero blocks out of the spread), or
// which holds an E8M0 NaN (0xFF), is left to a second kernel with an exact
// per-block path: each 32-element block's partial sum of unscaled
// codes is scaled with ldexp and added in fp32 (separate kernels keep the
// VALU-side accumulation out of the fast kernel's register budget).
#pragma once
#include <type_traits>

#include "mx_internal.h"

namespace mx {

// Operand rows are strided: row r of A's codes starts at a + r * lda and its
// scales at as + r * ldsa (bytes); the dense layout has lda = K (FP8) or K / 2
// (E2M1) and ldsa = K / 32.
struct GemmArgs {
    const uint8_t *a, *as, *b, *bs;
    void *c;
    int64_t ldc;
    int64_t lda, ldsa, ldb, ldsb;
    // K-panel layout of an operand's codes (pipelined kernels only): the 128
    // code bytes of row r that one stage reads, for K panel p, sit at
    // p * kp + r * 128; kp = 0 is the row layout above
    int64_t kpa = 0, kpb = 0;
    int M, N, K;
    int tiles_m, tiles_n;
};

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, NT = 256;
constexpr int kSpreadMax = 40;  // carrier fast path: per-row scale spread, binades

// compile-time loop: f(std::integral_constant<int, I>) for I in [I0, N)
template <int I, int N, class Fn>
__device__ __forceinline__ void static_for(Fn &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// byte offset of 16-byte chunk `ch` of row `row` in a swizzled LDS tile.
// 128-byte rows span 32 of the 64 banks, so two consecutive rows fill them;
// the key (row >> 1) & 7 gives the 16 rows that one pass of a 16-byte-per-lane
// read touches 16 different 4-bank groups.
template <int RB>
__device__ __forceinline__ int swz_key(int row) {
    if constexpr (RB == 128) return (row >> 1) & 7;
    else if constexpr (RB == 64) return (row >> 1) & 3;  // two rows per 128 bytes
    else return (row >> 2) & 1;                          // 32-byte rows: four rows per 128 bytes
}
template <int RB>
__device__ __forceinline__ int swz(int row, int ch) {
    return row * RB + ((ch ^ swz_key<RB>(row)) << 4);
}

// fp32 -> bf16, round to nearest even, NaN kept as a quiet NaN.  The
// gfx950 packed conversion (v_cvt_pk_bf16_f32, two values per instruction)
// does exactly that: on the device it equals the integer rounding
// (u + 0x7FFF + lsb) >> 16, with bit 6 set for NaN, on every one of the 2^32
// fp32 patterns, NaN payloads included -- and costs one instruction per pair
// instead of about six per value, which made the bf16 epilogue VALU-bound.
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{lo, hi}, v2bf));
}
__device__ __forceinline__ uint32_t bf16_rne(float f) { return bf16x2(f, 0.0f) & 0xFFFFu; }

// MI355X: 256 CUs in 8 XCDs, so an XCD runs 32 workgroups of one per CU at a time
constexpr int kCusPerXcd = 32;

// XCD-aware tile order: wg -> (tile row, tile column)
__device__ __forceinline__ void tile_of(const GemmArgs &g, int &m0, int &n0) {
    const int ntiles = g.tiles_m * g.tiles_n;
    const int wg = blockIdx.x;
    const int xcd = wg & 7, idx = wg >> 3;
    const int per = ntiles >> 3, rem = ntiles & 7;
    const int lt = xcd * per + (xcd < rem ? xcd : rem) + idx;
    constexpr int GROUP = 8;
    const int group_tiles = GROUP * g.tiles_n;
    const int grp = lt / group_tiles;
    const int first_m = grp * GROUP;
    const int gsz = (g.tiles_m - first_m) < GROUP ? (g.tiles_m - first_m) : GROUP;
    const int in_grp = lt - grp * group_tiles;
    m0 = (first_m + in_grp % gsz) * BM;
    n0 = (in_grp / gsz) * BN;
}

// Global -> register -> LDS staging of one K tile of codes (RBA / RBB bytes
// per row) and scales (SB bytes per row) for the A and B tiles.
template <int RBA, int RBB, int SB>
struct Stager {
    static constexpr int CPRA = RBA / 16, CPRB = RBB / 16;
    static constexpr int NLA = BM * CPRA / NT, NLB = BN * CPRB / NT;
    uint4 ra[NLA], rb[NLB];
    uint32_t rsa[SB / 4], rsb[SB / 4];

    __device__ __forceinline__ void load(const GemmArgs &g, int m0, int n0, int kt, int64_t rowA, int64_t rowB,
                                         int kblocks, bool scale_vec) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < NLA; i++) {
            const int id = tid + NT * i, row = id / CPRA, ch = id % CPRA;
            const int gr = min(m0 + row, g.M - 1);
            const int64_t off = (int64_t)kt * RBA + ch * 16;
            ra[i] = off < rowA ? *reinterpret_cast<const uint4 *>(g.a + gr * g.lda + off) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NLB; i++) {
            const int id = tid + NT * i, row = id / CPRB, ch = id % CPRB;
            const int gr = min(n0 + row, g.N - 1);
            const int64_t off = (int64_t)kt * RBB + ch * 16;
            rb[i] = off < rowB ? *reinterpret_cast<const uint4 *>(g.b + gr * g.ldb + off) : make_uint4(0, 0, 0, 0);
        }
        // scales: thread t owns row t of the A and B tiles
        const int ga = min(m0 + tid, g.M - 1), gb = min(n0 + tid, g.N - 1);
        const int kb0 = kt * SB;
        if (scale_vec && kb0 + SB <= kblocks) {
            if constexpr (SB == 4) {
                rsa[0] = *reinterpret_cast<const uint32_t *>(g.as + ga * g.ldsa + kb0);
                rsb[0] = *reinterpret_cast<const uint32_t *>(g.bs + gb * g.ldsb + kb0);
            } else {
                const uint2 ta = *reinterpret_cast<const uint2 *>(g.as + ga * g.ldsa + kb0);
                const uint2 tb = *reinterpret_cast<const uint2 *>(g.bs + gb * g.ldsb + kb0);
                rsa[0] = ta.x; rsa[1] = ta.y;
                rsb[0] = tb.x; rsb[1] = tb.y;
            }
        } else {
#pragma unroll
            for (int q = 0; q < SB / 4; q++) {
                uint32_t va = 0, vb = 0;
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const int kb = kb0 + 4 * q + t;
                    if (kb < kblocks) {
                        va |= (uint32_t)g.as[ga * g.ldsa + kb] << (8 * t);
                        vb |= (uint32_t)g.bs[gb * g.ldsb + kb] << (8 * t);
                    }
                }
                rsa[q] = va;
                rsb[q] = vb;
            }
        }
    }

    __device__ __forceinline__ void store(uint8_t *sA, uint8_t *sB, uint8_t *sAs, uint8_t *sBs) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < NLA; i++) {
            const int id = tid + NT * i, row = id / CPRA, ch = id % CPRA;
            *reinterpret_cast<uint4 *>(&sA[swz<RBA>(row, ch)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < NLB; i++) {
            const int id = tid + NT * i, row = id / CPRB, ch = id % CPRB;
            *reinterpret_cast<uint4 *>(&sB[swz<RBB>(row, ch)]) = rb[i];
        }
#pragma unroll
        for (int q = 0; q < SB / 4; q++) {
            reinterpret_cast<uint32_t *>(&sAs[tid * SB])[q] = rsa[q];
            reinterpret_cast<uint32_t *>(&sBs[tid * SB])[q] = rsb[q];
        }
    }
};

template <bool BF16OUT>
__device__ __forceinline__ void store_c(const GemmArgs &g, int m, int n, float v) {
    if (m < g.M && n < g.N) {
        if (BF16OUT)
            reinterpret_cast<uint16_t *>(g.c)[(int64_t)m * g.ldc + n] = (uint16_t)bf16_rne(v);
        else
            reinterpret_cast<float *>(g.c)[(int64_t)m * g.ldc + n] = v;
    }
}

// ---------------------------------------------------------------------------
// E2M1 x E2M1 on the block-scaled matrix instruction.
template <bool BF16OUT>
__global__ __launch_bounds__(NT, 1) void k_gemm_fp4(GemmArgs g) {
    constexpr int BK = 256, RB = 128, SB = 8, STEPS = 4;  // 256 FP4 = 128 bytes per row per tile
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * RB];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * RB];
    __shared__ __attribute__((aligned(16))) uint8_t sAs[2][BM * SB];
    __shared__ __attribute__((aligned(16))) uint8_t sBs[2][BN * SB];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    int m0, n0;
    tile_of(g, m0, n0);

    const int64_t rowA = g.K / 2, rowB = g.K / 2;
    const int kblocks = g.K / 32;
    const int ntk = (g.K + BK - 1) / BK;
    const bool scale_vec = (kblocks % SB == 0) && (((uintptr_t)g.as | (uintptr_t)g.bs) % SB == 0) &&
                           ((g.ldsa | g.ldsb) % SB == 0);

    Stager<RB, RB, SB> st;
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    auto compute = [&](int buf) {
        // per-lane scale words: byte 2s' of (word >> 8h) is block 2s' + h of the word
        uint32_t sa[4][2], sbw[4][2];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int ra_ = wm * 128 + i * 32 + l32, rb_ = wn * 128 + i * 32 + l32;
#pragma unroll
            for (int q = 0; q < 2; q++) {
                sa[i][q] = reinterpret_cast<const uint32_t *>(&sAs[buf][ra_ * SB])[q] >> (8 * h);
                sbw[i][q] = reinterpret_cast<const uint32_t *>(&sBs[buf][rb_ * SB])[q] >> (8 * h);
            }
        }
        static_for<0, STEPS>([&](auto step) {
            constexpr int s = decltype(step)::value;
            v8i fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint4 t = *reinterpret_cast<const uint4 *>(&sA[buf][swz<RB>(wm * 128 + i * 32 + l32, 2 * s + h)]);
                fa[i] = v8i{(int)t.x, (int)t.y, (int)t.z, (int)t.w, 0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint4 t = *reinterpret_cast<const uint4 *>(&sB[buf][swz<RB>(wn * 128 + j * 32 + l32, 2 * s + h)]);
                fb[j] = v8i{(int)t.x, (int)t.y, (int)t.z, (int)t.w, 0, 0, 0, 0};
            }
            constexpr int q = s / 2, sel = (2 * s) % 4;
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[i], fb[j], acc[i][j], 4, 4, sel, (int)sa[i][q], sel, (int)sbw[j][q]);
        });
    };

    st.load(g, m0, n0, 0, rowA, rowB, kblocks, scale_vec);
    st.store(sA[0], sB[0], sAs[0], sBs[0]);
    __syncthreads();
    for (int kt = 0; kt < ntk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < ntk) st.load(g, m0, n0, kt + 1, rowA, rowB, kblocks, scale_vec);
        compute(cur);
        if (kt + 1 < ntk) st.store(sA[cur ^ 1], sB[cur ^ 1], sAs[cur ^ 1], sBs[cur ^ 1]);
        __syncthreads();
    }

    // lane holds column n = l32 and rows 8(r/4) + 4h + r%4 of each 32 x 32 tile
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                store_c<BF16OUT>(g, m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3),
                                 n0 + wn * 128 + j * 32 + l32, acc[i][j][r]);
}

// ---------------------------------------------------------------------------
// bf16 carrier: any pair with an FP8 operand.

// 8 codes of one lane (bytes of `lo`, `hi` for FP8; nibbles of `lo` for E2M1)
// -> 8 bf16 = code * scale (scale a normal power of two: exact)
template <int F>
__device__ __forceinline__ v8bf to_bf16x8(uint32_t lo, uint32_t hi, float scale) {
    v2bf p0, p1, p2, p3;
    if constexpr (F == E4M3) {
        p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
        p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
        p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
        p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
    } else if constexpr (F == E5M2) {
        p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(lo, scale, false);
        p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(lo, scale, true);
        p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(hi, scale, false);
        p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(hi, scale, true);
    } else {
        p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(lo, scale, 0);
        p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(lo, scale, 1);
        p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(lo, scale, 2);
        p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(lo, scale, 3);
    }
    return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The codes a lane multiplies at step s (16 K per bf16 instruction): lane
// group h takes 16 consecutive codes of the step pair's 32-element block,
// the first 8 at the even step and the last 8 at the odd one.  A and B use
// the same order, so each instruction still pairs equal K, and both steps
// stay inside one block.  read_codes2 fetches both steps' codes at once: one
// 16-byte LDS read per lane (8 bytes for E2M1), whose 16-lane passes hit
// 16 different bank groups under the tile's swizzle.
template <int F, int RB>
__device__ __forceinline__ void read_codes(const uint8_t *tile, int row, int s, int h, uint32_t &lo, uint32_t &hi) {
    if constexpr (F == E2M1) {
        const int byte = 16 * (s >> 1) + 8 * h + 4 * (s & 1);  // 4 bytes
        lo = *reinterpret_cast<const uint32_t *>(&tile[swz<RB>(row, byte >> 4) + (byte & 15)]);
        hi = 0;
    } else {
        const int byte = 32 * (s >> 1) + 16 * h + 8 * (s & 1);  // 8 bytes
        const uint2 t = *reinterpret_cast<const uint2 *>(&tile[swz<RB>(row, byte >> 4) + (byte & 15)]);
        lo = t.x;
        hi = t.y;
    }
}
template <int F, int RB>
__device__ __forceinline__ uint4 read_codes2(const uint8_t *tile, int row, int j, int h) {
    if constexpr (F == E2M1) {
        const int byte = 16 * j + 8 * h;  // 8 bytes: steps 2j (x) and 2j + 1 (y)
        const uint2 t = *reinterpret_cast<const uint2 *>(&tile[swz<RB>(row, byte >> 4) + (byte & 15)]);
        return make_uint4(t.x, 0u, t.y, 0u);
    } else {
        const int byte = 32 * j + 16 * h;  // 16 bytes: steps 2j (x, y) and 2j + 1 (z, w)
        return *reinterpret_cast<const uint4 *>(&tile[swz<RB>(row, byte >> 4)]);
    }
}

// WIDE = false: the fast path, for tiles whose scales fit the carrier;
// WIDE = true: the exact per-block path, for the other tiles.  Both kernels
// are launched; each returns at once on the tiles that belong to the other.
template <int FA, int FB, bool BF16OUT, bool WIDE>
__global__ __launch_bounds__(NT, 1) void k_gemm_carrier(GemmArgs g) {
    constexpr int BK = 128, SB = 4, SUB = BK / 16;  // 16 K per bf16 instruction
    constexpr int RBA = FA == E2M1 ? 64 : 128, RBB = FB == E2M1 ? 64 : 128;
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * RBA];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * RBB];
    __shared__ __attribute__((aligned(16))) uint8_t sAs[2][BM * SB];
    __shared__ __attribute__((aligned(16))) uint8_t sBs[2][BN * SB];
    __shared__ int sRa[BM], sRb[BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    int m0, n0;
    tile_of(g, m0, n0);

    const int64_t rowA = FA == E2M1 ? g.K / 2 : g.K, rowB = FB == E2M1 ? g.K / 2 : g.K;
    const int kblocks = g.K / 32;
    const int ntk = (g.K + BK - 1) / BK;
    const bool scale_vec = (kblocks % SB == 0) && (((uintptr_t)g.as | (uintptr_t)g.bs) % SB == 0) &&
                           ((g.ldsa | g.ldsb) % SB == 0);

    // reference scales R = max over the row's blocks; the tile is "wide" if a
    // row's scales spread over more than kSpreadMax binades or hold 0xFF
    bool wide;
    {
        const int ga = min(m0 + tid, g.M - 1), gb = min(n0 + tid, g.N - 1);
        int amax = 0, amin = 255, bmax = 0, bmin = 255;
        const uint8_t *pa = g.as + ga * g.ldsa, *pb = g.bs + gb * g.ldsb;
        for (int kb = 0; kb < kblocks; kb++) {
            const int a = pa[kb], b = pb[kb];
            amax = max(amax, a); amin = min(amin, a);
            bmax = max(bmax, b); bmin = min(bmin, b);
        }
        sRa[tid] = amax;
        sRb[tid] = bmax;
        const bool w = amax - amin > kSpreadMax || bmax - bmin > kSpreadMax || amax == 255 || bmax == 255;
        wide = __syncthreads_or(w) != 0;
    }
    if (wide != WIDE) return;  // uniform across the workgroup

    Stager<RBA, RBB, SB> st;
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    // fast path: a' = code * 2^(S - R) for this lane's row, 4 blocks per tile
    auto compute_fast = [&](int buf) {
        float sca[4][4], scb[4][4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int ra_ = wm * 128 + i * 32 + l32, rb_ = wn * 128 + i * 32 + l32;
            const uint32_t wa = *reinterpret_cast<const uint32_t *>(&sAs[buf][ra_ * SB]);
            const uint32_t wb = *reinterpret_cast<const uint32_t *>(&sBs[buf][rb_ * SB]);
            const int Ra = sRa[ra_], Rb = sRb[rb_];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                sca[i][q] = __builtin_amdgcn_ldexpf(1.0f, (int)((wa >> (8 * q)) & 0xFF) - Ra);
                scb[i][q] = __builtin_amdgcn_ldexpf(1.0f, (int)((wb >> (8 * q)) & 0xFF) - Rb);
            }
        }
#pragma unroll
        for (int s = 0; s < SUB; s++) {
            v8bf fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                uint32_t lo, hi;
                read_codes<FA, RBA>(sA[buf], wm * 128 + i * 32 + l32, s, h, lo, hi);
                fa[i] = to_bf16x8<FA>(lo, hi, sca[i][s >> 1]);
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                uint32_t lo, hi;
                read_codes<FB, RBB>(sB[buf], wn * 128 + j * 32 + l32, s, h, lo, hi);
                fb[j] = to_bf16x8<FB>(lo, hi, scb[j][s >> 1]);
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };

    // exact path: per block, partial sum of unscaled codes, then ldexp by S_a + S_b
    // (the block loop stays rolled to bound register pressure; only the tile
    // loops that index the accumulators are unrolled)
    auto compute_wide = [&](int buf) {
#pragma unroll 1
        for (int blk = 0; blk < BK / 32; blk++) {
            static_for<0, 4>([&](auto ii) {
                constexpr int i = decltype(ii)::value;
                int sa_r[16];
#pragma unroll
                for (int r = 0; r < 16; r++)
                    sa_r[r] = sAs[buf][(wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * SB + blk];
                static_for<0, 4>([&](auto jj) {
                    constexpr int j = decltype(jj)::value;
                    v16f p;
#pragma unroll
                    for (int r = 0; r < 16; r++) p[r] = 0.f;
#pragma unroll
                    for (int s = 0; s < 2; s++) {
                        uint32_t lo, hi;
                        read_codes<FA, RBA>(sA[buf], wm * 128 + i * 32 + l32, 2 * blk + s, h, lo, hi);
                        const v8bf a8 = to_bf16x8<FA>(lo, hi, 1.0f);
                        read_codes<FB, RBB>(sB[buf], wn * 128 + j * 32 + l32, 2 * blk + s, h, lo, hi);
                        const v8bf b8 = to_bf16x8<FB>(lo, hi, 1.0f);
                        p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a8, b8, p, 0, 0, 0);
                    }
                    const int sb = sBs[buf][(wn * 128 + j * 32 + l32) * SB + blk];
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        // an E8M0 NaN scale makes the term NaN (a select on the bit pattern)
                        const uint32_t v = __float_as_uint(__builtin_amdgcn_ldexpf(p[r], sa_r[r] + sb - 254));
                        acc[i][j][r] += __uint_as_float((sa_r[r] == 255 || sb == 255) ? 0x7FC00000u : v);
                    }
                });
            });
        }
    };

    st.load(g, m0, n0, 0, rowA, rowB, kblocks, scale_vec);
    st.store(sA[0], sB[0], sAs[0], sBs[0]);
    __syncthreads();
    for (int kt = 0; kt < ntk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < ntk) st.load(g, m0, n0, kt + 1, rowA, rowB, kblocks, scale_vec);
        if constexpr (WIDE)
            compute_wide(cur);
        else
            compute_fast(cur);
        if (kt + 1 < ntk) st.store(sA[cur ^ 1], sB[cur ^ 1], sAs[cur ^ 1], sBs[cur ^ 1]);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int nl = wn * 128 + j * 32 + l32;
            const int Rb = sRb[nl];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int ml = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                const float v = WIDE ? acc[i][j][r] : __builtin_amdgcn_ldexpf(acc[i][j][r], sRa[ml] + Rb - 254);
                store_c<BF16OUT>(g, m0 + ml, n0 + nl, v);
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Pipelined kernels (K a whole number of stages, aligned pointers): the same
// tiling and arithmetic as above, restructured for gfx950's memory system.
//   - Operand tiles move with BUFFER_LOAD ... LDS (global memory straight to
//     LDS, no register staging).  A stage holds 128 code bytes per row (256
//     E2M1 or 128 FP8 elements; 64 bytes for an E2M1 operand paired with FP8):
//     every row request then covers whole 128-byte L2 lines, which measured
//     twice the L2 throughput of 64-byte slices.  Two stages (2 x 68 KiB of
//     LDS): one loads while the other is multiplied.
//   - Each stage has its own LDS arrays and the loop is unrolled by the stage
//     count, so stage indices are compile-time; every stage load is issued
//     unconditionally (past the last tile its offset points outside the
//     buffer and the load returns zeros).  This keeps the compiler's
//     wait-count tracking exact, and rows past M or N read as zeros through
//     the buffer's range check.
//   - The matrix instructions run with B as the first operand, so a lane's
//     accumulators hold four consecutive columns of one row of C.  The
//     epilogue stages each wave's 128 x 128 tile of C through the (then idle)
//     LDS stage buffers and writes whole 256-byte row segments.
namespace pipe {

typedef __attribute__((address_space(3))) void *lds_t;
constexpr int NS = 2;

// Workgroup barrier without the compiler's implied vmcnt(0): the stage loads
// are waited for explicitly.  LDS reads this wave issued before the barrier
// are drained first (lgkmcnt(0)): the compiler may leave them in flight past
// an inline-asm barrier, after which other waves' DMA may overwrite the buffer.
// The scheduling fences keep register-only work (MFMAs) on its side of the
// barrier, so one stage's fragments are never live across it.
__device__ __forceinline__ void barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// tile hand-over mark between the carrier's fast and exact kernels (see there)
constexpr uint16_t kMarkBf16 = 0x7FBE;      // bf16 NaN, quiet bit clear: the conversion never yields it
constexpr uint32_t kMarkF32 = 0x7FBADBADu;  // fp32 NaN, quiet bit clear: arithmetic never yields it
template <bool BF16OUT>
__device__ __forceinline__ void mark_tile(const GemmArgs &g, int m0, int n0) {
    const int64_t i = (int64_t)m0 * g.ldc + n0;
    if constexpr (BF16OUT) reinterpret_cast<uint16_t *>(g.c)[i] = kMarkBf16;
    else reinterpret_cast<uint32_t *>(g.c)[i] = kMarkF32;
}
template <bool BF16OUT>
__device__ __forceinline__ bool tile_marked(const GemmArgs &g, int m0, int n0) {
    const int64_t i = (int64_t)m0 * g.ldc + n0;
    if constexpr (BF16OUT) return reinterpret_cast<const uint16_t *>(g.c)[i] == kMarkBf16;
    else return reinterpret_cast<const uint32_t *>(g.c)[i] == kMarkF32;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Raw buffer descriptor: base address, no stride, `bytes` records (reads at
// or past the end return zeros), dword data format.
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return v4i{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

// 16 bytes per lane from buffer r at voff + soff straight into LDS: lane l
// lands at lds + 16 l.  Written as inline asm so that the compiler's own
// wait-count tracking, which cannot always tell the stage buffers apart and
// would then wait for every load in flight before an LDS read, stays out of
// it: the kernel waits for the loads explicitly (vmcnt) before its barriers.
// M0 carries the LDS address and needs one wait state before the load.
__device__ __forceinline__ void dma16(v4i r, void *lds, int voff, int soff) {
    const uint32_t m = (uint32_t)(uintptr_t)(lds_t)lds;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, %3 offen lds"
                 :
                 : "v"(voff), "s"(m), "s"(r), "s"(soff)
                 : "memory", "m0");
}

// Largest of a row's E8M0 bytes, smallest of its nonzero ones (255 if none)
// and whether any is zero.  With vec (16-byte aligned, n % 16 == 0) the bytes
// come as uint4 loads, four in flight at a time: the scan runs once per tile
// and row, before the tile's first stage.
__device__ __forceinline__ void row_scale_range(const uint8_t *p, int n, bool vec, int &mx, int &mnz, bool &has0) {
    mx = 0;
    mnz = 255;
    has0 = false;
    const auto take = [&](int b) {
        mx = max(mx, b);
        if (b) mnz = min(mnz, b);
        else has0 = true;
    };
    const auto take16 = [&](const uint4 &t) {
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int q = 0; q < 16; q++) take((w[q >> 2] >> (8 * (q & 3))) & 0xFF);
    };
    if (vec) {
        int k = 0;
        for (; k + 64 <= n; k += 64) {
            uint4 t[4];
#pragma unroll
            for (int u = 0; u < 4; u++) t[u] = *reinterpret_cast<const uint4 *>(p + k + 16 * u);
#pragma unroll
            for (int u = 0; u < 4; u++) take16(t[u]);
        }
        for (; k < n; k += 16) take16(*reinterpret_cast<const uint4 *>(p + k));
    } else {
        for (int k = 0; k < n; k++) take(p[k]);
    }
}

// true if every block of the row whose scale byte is 0 holds only zero codes
// (either sign: MAG masks the magnitude bits): codes c of the row (16-byte
// aligned; with kp != 0 the row's bytes of K panel 0, see GemmArgs), scales p,
// n blocks of BB code bytes
template <int BB, uint32_t MAG>
__device__ __forceinline__ bool zero_blocks_clear(const uint8_t *c, const uint8_t *p, int n, bool vec, int64_t kp) {
    uint32_t any = 0;
    const auto check = [&](int k) {
        const int64_t pos = (int64_t)k * BB;
        const uint8_t *blk = kp ? c + (pos >> 7) * kp + (pos & 127) : c + pos;
#pragma unroll
        for (int q = 0; q < BB; q += 16) {
            const uint4 t = *reinterpret_cast<const uint4 *>(blk + q);
            any |= (t.x | t.y | t.z | t.w) & MAG;
        }
    };
    if (vec) {
        for (int k = 0; k < n; k += 16) {
            const uint4 t = *reinterpret_cast<const uint4 *>(p + k);
            const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int q = 0; q < 16; q++)
                if (((w[q >> 2] >> (8 * (q & 3))) & 0xFF) == 0) check(k + q);
        }
    } else {
        for (int k = 0; k < n; k++)
            if (p[k] == 0) check(k);
    }
    return any == 0;
}

// four consecutive columns n .. n+3 of row m
template <bool BF16OUT>
__device__ __forceinline__ void store_c4(const GemmArgs &g, int m, int n, float v0, float v1, float v2, float v3,
                                         bool vec) {
    if (m >= g.M) return;
    if (vec && n + 3 < g.N) {
        if constexpr (BF16OUT) {
            const uint32_t lo = bf16x2(v0, v1), hi = bf16x2(v2, v3);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(g.c) + (int64_t)m * g.ldc + n) = make_uint2(lo, hi);
        } else {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(g.c) + (int64_t)m * g.ldc + n) =
                make_float4(v0, v1, v2, v3);
        }
    } else {
        store_c<BF16OUT>(g, m, n, v0);
        store_c<BF16OUT>(g, m, n + 1, v1);
        store_c<BF16OUT>(g, m, n + 2, v2);
        store_c<BF16OUT>(g, m, n + 3, v3);
    }
}

// MODE 0: E2M1 x E2M1, block-scaled instruction.  MODE 1: carrier fast path.
// MODE 2: carrier exact per-block path (tiles the fast path leaves).
// 512 threads: 8 waves, two per SIMD, each a 128 x 64 tile of C (4 x 2 tiles
// of 32 x 32, 128 accumulators), so one wave multiplies while the other
// waits on LDS, the barrier or the stage loads.
constexpr int PNT = 512;
template <int FA, int FB, bool BF16OUT, int MODE>
__global__ __launch_bounds__(PNT, 1) void k_gemm_pipe(GemmArgs g) {
    constexpr bool A4 = FA == E2M1, B4 = FB == E2M1;
    constexpr int KE = (A4 && B4) ? 256 : 128;         // K elements per stage
    constexpr int RBA = A4 ? KE / 2 : KE, RBB = B4 ? KE / 2 : KE;
    constexpr int SBY = KE / 32;                       // scale bytes per row per stage: 8 or 4
    constexpr int NSW = SBY / 4;                       // scale words per row per stage
    constexpr int SPS = 16 / SBY;                      // stages per scale slot (16 scale bytes per row)
    constexpr int NW = PNT / 64;                       // waves
    // All eight waves share the stage loads.  (Leaving them to one wave per
    // SIMD, so that its partner multiplies meanwhile, measured slower on the
    // gate/up projection GEMM: 629 us against 563 us.)
    constexpr int NWD = 8;
    constexpr int NIA = BM * RBA / 1024 / NWD, NIB = BN * RBB / 1024 / NWD;  // 1 KiB DMA per wave instruction
    constexpr int CPRA = RBA / 16, CPRB = RBB / 16;
    static_assert(NIA >= 1 && NIB >= 1, "DMA split");
    static_assert(NW == 8 && NWD == NW && BM == 256 && BN == 256, "load split");

    // Code stages alternate between two buffers; scale slots (16 bytes per
    // row: the scales of SPS consecutive stages) alternate between two more.
    // Every buffer is a separate LDS object selected at compile time, so the
    // compiler can see that a stage load never aliases the buffer being read.
    __shared__ __attribute__((aligned(16))) uint8_t sA0[BM * RBA], sA1[BM * RBA];
    __shared__ __attribute__((aligned(16))) uint8_t sB0[BN * RBB], sB1[BN * RBB];
    __shared__ __attribute__((aligned(16))) uint8_t sS0[2][BM * 16], sS1[2][BM * 16];  // [A, B][row * 16 + byte]
    __shared__ int sRa[BM], sRb[BN];
    auto stA = [&](auto S) -> uint8_t * { if constexpr (decltype(S)::value == 0) return sA0; else return sA1; };
    auto stB = [&](auto S) -> uint8_t * { if constexpr (decltype(S)::value == 0) return sB0; else return sB1; };
    auto stS = [&](auto T, int op) -> uint8_t * { if constexpr (decltype(T)::value == 0) return sS0[op]; else return sS1[op]; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS DMA bases go through M0
    const int wm = wave >> 2, wn = wave & 3;  // wave tile: rows wm*128 .. +127, cols wn*64 .. +63
    const int l32 = lane & 31, h = lane >> 5;
    int m0, n0;
    tile_of(g, m0, n0);
    // Every other round of an XCD's tiles takes K's scale slots in reverse order (the stages
    // inside a slot stay in order).  Consecutive rounds share the XCD's A rows, and a round
    // then starts on the slots the round before read last, which are still in L2: the
    // gate/up projection GEMM fetches 558 MB instead of 722 MB from beyond L2.  Only the
    // order of the fp32 sum over K changes.
    const bool krev = ((blockIdx.x >> 3) / kCusPerXcd) & 1;

    // row strides in bytes (the launcher keeps 256 rows of either operand below 2^31 bytes);
    // a K-panel operand has rows of one stage's RB = 128 bytes, and stage kt in panel kt
    const int rowA = g.kpa ? RBA : (int)g.lda, rowB = g.kpb ? RBB : (int)g.ldb;
    const int srowA = (int)g.ldsa, srowB = (int)g.ldsb;
    const int kblocks = g.K / 32;
    const int ntk = g.K / KE;
    const int mrows = min(BM, g.M - m0), nrows = min(BN, g.N - n0);
    // a K-panel operand's record range runs to the end of its codes (rows past M in a panel
    // are the next panel's first rows: they only reach rows of C past M, which are not stored)
    const uint32_t nrecA = g.kpa ? (uint32_t)((int64_t)ntk * g.kpa - (int64_t)m0 * RBA) : (uint32_t)mrows * rowA;
    const uint32_t nrecB = g.kpb ? (uint32_t)((int64_t)ntk * g.kpb - (int64_t)n0 * RBB) : (uint32_t)nrows * rowB;
    const int stA_ = g.kpa ? (int)g.kpa : RBA, stB_ = g.kpb ? (int)g.kpb : RBB;  // bytes per stage
    const uint32_t nrecSA = (uint32_t)mrows * srowA, nrecSB = (uint32_t)nrows * srowB;
    const v4i rA = rsrc(g.a + (int64_t)m0 * rowA, nrecA);
    const v4i rB = rsrc(g.b + (int64_t)n0 * rowB, nrecB);
    const v4i rSA = rsrc(g.as + (int64_t)m0 * srowA, nrecSA);
    const v4i rSB = rsrc(g.bs + (int64_t)n0 * srowB, nrecSB);

    // carrier: reference scale per row and the tile's path (threads 0..255:
    // rows of A, 256..511: rows of B).  The fast kernel (MODE 1) leaves a tile
    // whose rows' scales spread too far (or hold 0xFF) to the exact per-block
    // kernel (MODE 2) and marks it with a sentinel in C[m0][n0] that no result
    // store produces (a NaN with its quiet bit clear); the exact kernel, which
    // runs next on the same stream, reads that one element instead of every
    // scale of the tile.  A false match would only make it recompute a tile,
    // exactly.
    if constexpr (MODE == 2) {
        if (!tile_marked<BF16OUT>(g, m0, n0)) return;  // uniform across the workgroup
    }
    if constexpr (MODE == 1) {
        const bool isA = tid < BM;
        const int r = isA ? tid : tid - BM;
        const int gr = isA ? min(m0 + r, g.M - 1) : min(n0 + r, g.N - 1);
        const bool vec = (kblocks % 16 == 0) && ((((uintptr_t)g.as | (uintptr_t)g.bs) & 15) == 0) &&
                         (((srowA | srowB) & 15) == 0);
        int mx_, mn_;
        bool has0;
        const uint8_t *ps = (isA ? g.as : g.bs) + (int64_t)gr * (isA ? srowA : srowB);
        row_scale_range(ps, kblocks, vec, mx_, mn_, has0);
        (isA ? sRa : sRb)[r] = mx_;
        bool w = mx_ - mn_ > kSpreadMax || mx_ == 255;
        if (has0 && mx_ > kSpreadMax && !w) {
            // A block with scale byte 0 beside blocks more than kSpreadMax binades
            // above it.  If its codes are all zero it adds exactly 0 under any finite
            // scale; its rebased byte 127 - R stays in [0, 127] (a finite scale, no
            // borrow into the neighbouring bytes of the scale word) as long as
            // R <= 127.  Then the tile keeps the fast path; a block of genuinely tiny
            // values (nonzero codes under scale byte 0) sends it to the exact kernel.
            const uint8_t *pc = isA ? g.a + (int64_t)gr * rowA : g.b + (int64_t)gr * rowB;
            const int64_t kp = isA ? g.kpa : g.kpb;
            w = mx_ > 127 || !((isA ? A4 : B4) ? zero_blocks_clear<16, 0x77777777u>(pc, ps, kblocks, vec, kp)
                                                : zero_blocks_clear<32, 0x7F7F7F7Fu>(pc, ps, kblocks, vec, kp));
        }
        if (__syncthreads_or(w) != 0) {  // uniform across the workgroup
            if (tid == 0) mark_tile<BF16OUT>(g, m0, n0);
            return;
        }
    }

    // per-lane DMA source offsets, constant along K: lane l of instruction q
    // fills LDS bytes [16 l, 16 l + 16) of its 1 KiB segment = physical chunk
    // l % CPR of row seg * (64 / CPR) + l / CPR, i.e. logical chunk pch ^ key.
    // Instruction q's rows are instruction 0's plus q * 64 / CPR: the row part
    // is a uniform (scalar) offset, and the swizzle key of 128-byte rows moves
    // by 8 rows -> key ^ 4 on odd q; the keys of 64- and 32-byte rows do not
    // change.
    static_assert(64 / CPRA == 8 || RBA < 128, "8 rows per instruction");
    static_assert(64 / CPRB == 8 || RBB < 128, "8 rows per instruction");
    const int dw = wave;  // index among the loading waves
    const int rowA0 = dw * NIA * (64 / CPRA) + lane / CPRA, rowB0 = dw * NIB * (64 / CPRB) + lane / CPRB;
    const int keyA = swz_key<RBA>(rowA0), keyB = swz_key<RBB>(rowB0);
    const int keyA1 = RBA == 128 ? (keyA ^ 4) : keyA, keyB1 = RBB == 128 ? (keyB ^ 4) : keyB;
    const int voffA = rowA0 * rowA + (((lane % CPRA) ^ keyA) << 4);
    const int voffB = rowB0 * rowB + (((lane % CPRB) ^ keyB) << 4);
    const int voffA1 = rowA0 * rowA + (((lane % CPRA) ^ keyA1) << 4);
    const int voffB1 = rowB0 * rowB + (((lane % CPRB) ^ keyB1) << 4);

    // scale slot loads: eight 64-row instructions (four for A's rows, four
    // for B's), NSI per loading wave; 16 bytes of each row, one line per row
    constexpr int NSI = 8 / NWD;
    const int sop = (dw * NSI) >> 2;
    const int srow0 = ((dw * NSI) & 3) * 64;
    const int sstride = sop ? srowB : srowA;  // uniform: the operand this wave loads
    const int svoff = (srow0 + lane) * sstride;

    // codes of stage kt into code buffer S; with SCALES, also the scales of
    // stages kt .. kt + SPS - 1 into scale slot T.  Past the last stage the
    // offsets point beyond the buffers' records, which reads zeros.
    auto issue = [&](auto S, auto T, auto SCALES, int kt) {
        const bool live = kt < ntk;
        const int pk = krev ? (ntk - SPS - kt / SPS * SPS + kt % SPS) : kt;  // stage of K loaded
        const int soA = live ? pk * stA_ : (int)nrecA, soB = live ? pk * stB_ : (int)nrecB;
#pragma unroll
        for (int q = 0; q < NIA; q++)
            dma16(rA, stA(S) + (dw * NIA + q) * 1024, (q & 1) ? voffA1 : voffA, soA + q * (64 / CPRA) * rowA);
#pragma unroll
        for (int q = 0; q < NIB; q++)
            dma16(rB, stB(S) + (dw * NIB + q) * 1024, (q & 1) ? voffB1 : voffB, soB + q * (64 / CPRB) * rowB);
        // branch-free (uniform selects, EXEC masks): a branch would split the
        // loop body into blocks, and the compiler would then sink each stage's
        // MFMAs into the block of their next use, past the barrier
        if constexpr (decltype(SCALES)::value) {
#pragma unroll
            for (int u = 0; u < NSI; u++)
                dma16(sop ? rSB : rSA, stS(T, sop) + (srow0 + 64 * u) * 16, svoff + 64 * u * sstride,
                      live ? pk * SBY : (int)(sop ? nrecSB : nrecSA));
        }
    };

    v16f acc[4][2];  // acc[i][j]: C^T tile of A rows i, B rows j
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    // stage held in code buffer S whose scales are bytes SBY * P .. of slot T;
    // issue_next() sends the next stage's loads (to the other buffer) once this
    // stage's first LDS reads are out, so that their issue overlaps the reads'
    // latency instead of delaying them
    auto compute = [&](auto S, auto T, auto P, bool cur_live, auto &&issue_next) {
        const uint8_t *tA = stA(S), *tB = stB(S);
        const uint8_t *tSA = stS(T, 0) + SBY * decltype(P)::value, *tSB = stS(T, 1) + SBY * decltype(P)::value;
        if constexpr (MODE == 0) {
            // scale words of a row: blocks 4w .. 4w+3 of the stage; >> 8h leaves
            // this lane's blocks 4w + h and 4w + 2 + h at bytes 0 and 2
            uint32_t sa[4][NSW], sbw[2][NSW];
#pragma unroll
            for (int w = 0; w < NSW; w++) {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    sa[i][w] = *reinterpret_cast<const uint32_t *>(&tSA[(wm * 128 + i * 32 + l32) * 16 + 4 * w]) >> (8 * h);
#pragma unroll
                for (int j = 0; j < 2; j++)
                    sbw[j][w] = *reinterpret_cast<const uint32_t *>(&tSB[(wn * 64 + j * 32 + l32) * 16 + 4 * w]) >> (8 * h);
            }
            // Fragments are double-buffered: step s + 1's LDS reads are issued
            // before step s's MFMAs, and a scheduling fence closes each step,
            // so at most two steps' fragments are live beside the accumulators.
            uint4 fa[2][4], fb[2][2];
            auto load = [&](auto step) {
                constexpr int s = decltype(step)::value, b = s & 1;
#pragma unroll
                for (int i = 0; i < 4; i++)
                    fa[b][i] = *reinterpret_cast<const uint4 *>(&tA[swz<RBA>(wm * 128 + i * 32 + l32, 2 * s + h)]);
#pragma unroll
                for (int j = 0; j < 2; j++)
                    fb[b][j] = *reinterpret_cast<const uint4 *>(&tB[swz<RBB>(wn * 64 + j * 32 + l32, 2 * s + h)]);
            };
            load(std::integral_constant<int, 0>{});
            issue_next();
            static_for<0, KE / 64>([&](auto step) {
                constexpr int s = decltype(step)::value, b = s & 1;
                constexpr int w = s / 2, sel = (2 * s) % 4;
                if constexpr (s + 1 < KE / 64) load(std::integral_constant<int, s + 1>{});
#pragma unroll
                for (int i = 0; i < 4; i++)
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        const uint4 x = fa[b][i], y = fb[b][j];
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            v8i{(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0},
                            v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0}, acc[i][j], 4, 4, sel,
                            (int)sbw[j][w], sel, (int)sa[i][w]);
                    }
                // pin the order: left to itself the scheduler sank step s + 1's reads below
                // six of step s's MFMAs, and step s + 1 then waited on their LDS latency
                if constexpr (s + 1 < KE / 64) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // the six LDS reads
                    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // then the eight MFMAs
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        } else if constexpr (MODE == 1) {
            // Per row, the stage's four block exponents rebased on the row's reference:
            // byte q = S_q - R + 127, which lies in [87, 127] for real blocks (scale spread
            // <= 40 binades, S_q <= R; an all-zero block under byte 0 only stays on this
            // path while R <= 127), so 2^(S_q - R) <= 1 is the float with that byte as its
            // exponent field.  A stage past the end of K holds zero codes and zero scale
            // bytes, whose rebased bytes would wrap (255 is Inf, and 0 * Inf a NaN): it
            // takes scale 1 instead, so its terms add exactly 0.  Rows past the edge of
            // the matrix may wrap too, but they only reach rows and columns of C that are
            // not stored.
            const auto rebase = [](uint32_t w, int R) -> uint32_t {
                const uint32_t rr = __builtin_amdgcn_perm(0u, (uint32_t)R, 0u);  // R in every byte
                return w - rr + 0x7F7F7F7Fu;  // bytewise S_q + 127 - R, no carries for real blocks
            };
            const auto block_scale = [](uint32_t d, int q) -> float {
                return __uint_as_float(((d >> (8 * q)) & 0xFFu) << 23);
            };
            uint32_t da[4], db[2];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int ra_ = wm * 128 + i * 32 + l32;
                const uint32_t d = rebase(*reinterpret_cast<const uint32_t *>(&tSA[ra_ * 16]), sRa[ra_]);
                da[i] = cur_live ? d : 0x7F7F7F7Fu;
            }
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int rb_ = wn * 64 + j * 32 + l32;
                const uint32_t d = rebase(*reinterpret_cast<const uint32_t *>(&tSB[rb_ * 16]), sRb[rb_]);
                db[j] = cur_live ? d : 0x7F7F7F7Fu;
            }
            // Software-pipelined: the codes of a step pair are read from LDS (one 16-byte
            // read per fragment) at the top of the step before the pair, and step t + 1's
            // fragments are converted in the shadow of step t's MFMAs.  The MFMAs go column by
            // column: the four on B fragment 0 first (they cover the LDS latency), then B
            // fragment 0 of step t + 1 is converted into the registers they released, and
            // each A fragment of step t + 1 right after the last MFMA that reads its
            // predecessor, so about one step of fragments is live at a time.  (Converted
            // just before their own MFMAs, with both waves of a SIMD released by the same
            // barrier, the conversions and the matrix work had run one after the other.)
            v8bf fa[4], fb[2];
            uint4 ca[4], cb[2];  // codes of the current step pair
            const auto rd = [&](int j) {
#pragma unroll
                for (int jj = 0; jj < 2; jj++) cb[jj] = read_codes2<FB, RBB>(tB, wn * 64 + jj * 32 + l32, j, h);
#pragma unroll
                for (int i = 0; i < 4; i++) ca[i] = read_codes2<FA, RBA>(tA, wm * 128 + i * 32 + l32, j, h);
            };
            const auto lo_of = [](const uint4 &c, int odd) { return odd ? c.z : c.x; };
            const auto hi_of = [](const uint4 &c, int odd) { return odd ? c.w : c.y; };
            rd(0);
            issue_next();
#pragma unroll
            for (int i = 0; i < 4; i++) fa[i] = to_bf16x8<FA>(ca[i].x, ca[i].y, block_scale(da[i], 0));
#pragma unroll
            for (int j = 0; j < 2; j++) fb[j] = to_bf16x8<FB>(cb[j].x, cb[j].y, block_scale(db[j], 0));
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, KE / 16>([&](auto step) {
                constexpr int t = decltype(step)::value;
                constexpr bool more = t + 1 < KE / 16;
                constexpr int odd = (t + 1) & 1;  // step t + 1 takes the second half of its pair
                if constexpr (more && odd == 0) rd((t + 1) >> 1);
#pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[0], fa[i], acc[i][0], 0, 0, 0);
                if constexpr (more) fb[0] = to_bf16x8<FB>(lo_of(cb[0], odd), hi_of(cb[0], odd), block_scale(db[0], (t + 1) >> 1));
                __builtin_amdgcn_sched_barrier(0);
                static_for<0, 4>([&](auto ii) {
                    constexpr int i = decltype(ii)::value;
                    acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1], fa[i], acc[i][1], 0, 0, 0);
                    if constexpr (more) fa[i] = to_bf16x8<FA>(lo_of(ca[i], odd), hi_of(ca[i], odd), block_scale(da[i], (t + 1) >> 1));
                    __builtin_amdgcn_sched_barrier(0);
                });
                if constexpr (more) fb[1] = to_bf16x8<FB>(lo_of(cb[1], odd), hi_of(cb[1], odd), block_scale(db[1], (t + 1) >> 1));
                __builtin_amdgcn_sched_barrier(0);
            });
        } else {
            issue_next();
#pragma unroll 1
            for (int blk = 0; blk < KE / 32; blk++) {
                static_for<0, 2>([&](auto jj) {
                    constexpr int j = decltype(jj)::value;
                    int sb_r[16];  // scale of column n = 8(r/4) + 4h + r%4 of tile j
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        sb_r[r] = tSB[(wn * 64 + j * 32 + 8 * (r >> 2) + 4 * h + (r & 3)) * 16 + blk];
                    static_for<0, 4>([&](auto ii) {
                        constexpr int i = decltype(ii)::value;
                        v16f p;
#pragma unroll
                        for (int r = 0; r < 16; r++) p[r] = 0.f;
#pragma unroll
                        for (int t = 0; t < 2; t++) {
                            uint32_t lo, hi;
                            read_codes<FA, RBA>(tA, wm * 128 + i * 32 + l32, 2 * blk + t, h, lo, hi);
                            const v8bf a8 = to_bf16x8<FA>(lo, hi, 1.0f);
                            read_codes<FB, RBB>(tB, wn * 64 + j * 32 + l32, 2 * blk + t, h, lo, hi);
                            const v8bf b8 = to_bf16x8<FB>(lo, hi, 1.0f);
                            p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b8, a8, p, 0, 0, 0);
                        }
                        const int sa = tSA[(wm * 128 + i * 32 + l32) * 16 + blk];
#pragma unroll
                        for (int r = 0; r < 16; r++) {
                            // an E8M0 NaN scale makes the term NaN: a select on the bit pattern
                            // (written as a conditional on floats, the compiler branched here and
                            // spilled ~1800 registers around the branches)
                            const uint32_t v = __float_as_uint(__builtin_amdgcn_ldexpf(p[r], sa + sb_r[r] - 254));
                            const uint32_t nan_or_v = (sa == 255 || sb_r[r] == 255) ? 0x7FC00000u : v;
                            acc[i][j][r] += __uint_as_float(nan_or_v);
                        }
                    });
                });
            }
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<bool, true>;
    issue(I0{}, I0{}, B1{}, 0);
    for (int kt0 = 0; kt0 < ntk; kt0 += 2 * SPS) {
        // stage kt0 + u sits in code buffer u % 2 and scale slot u / SPS.
        // After the barrier every wave is done with stage kt0 + u - 1, whose
        // code buffer receives the next stage (and, at a slot boundary, whose
        // scale slot receives the next SPS stages' scales).
        static_for<0, 2 * SPS>([&](auto uu) {
            constexpr int u = decltype(uu)::value;
            const int kt = kt0 + u;  // stage computed in this step
            wait_vm<0>();  // this stage's loads
            barrier();
            // unconditional: a stage past the end holds zero codes and zero
            // scale bytes (out-of-range loads), which add exactly 0; a branch
            // here would let the compiler sink the stage's MFMAs past the next
            // barrier and keep every fragment of the stage live across it
            compute(std::integral_constant<int, u % 2>{}, std::integral_constant<int, u / SPS>{},
                    std::integral_constant<int, u % SPS>{}, kt < ntk, [&] {
                        issue(std::integral_constant<int, (u + 1) % 2>{},
                              std::integral_constant<int, ((u + 1) / SPS) % 2>{},
                              std::integral_constant<bool, (u + 1) % SPS == 0>{}, kt + 1);
                    });
        });
    }
    wait_vm<0>();  // drain the out-of-range stage loads before the workgroup ends

    // lane: row m = i*32 + l32 of the wave's tile, columns 8(r/4) + 4h + r%4 of tile j
    auto value = [&](int i, int j, int q, int e) -> float {
        float v = acc[i][j][4 * q + e];
        if constexpr (MODE == 1) v = __builtin_amdgcn_ldexpf(v, sRa[wm * 128 + i * 32 + l32] +
                                                                  sRb[wn * 64 + j * 32 + 8 * q + 4 * h + e] - 254);
        return v;
    };
    if constexpr (RBA == 128 || RBB == 128) {
        // Stage the wave's 128 x 64 tile of C through LDS (the stage buffers,
        // free once every wave has left the main loop) and write it back with
        // consecutive lanes covering whole 128-byte (bf16) or 256-byte (fp32)
        // row segments.  16-byte chunks are XOR-swizzled by the row so the
        // column-wise writes spread over the banks.  With 128-byte rows in
        // both operands' stage buffers every wave has 16 KiB (bf16 in one pass
        // of 128 rows, fp32 in two of 64); with one E2M1 operand (64-byte rows)
        // the two 32 KiB buffers of the other give each wave 8 KiB (passes of
        // 64 or 32 rows).
        barrier();
        constexpr int REG = (RBA == 128 && RBB == 128) ? 16384 : 8192;  // bytes per wave
        uint8_t *reg;
        if constexpr (REG == 16384)
            reg = ((wave >> 1) == 0 ? sA0 : (wave >> 1) == 1 ? sA1 : (wave >> 1) == 2 ? sB0 : sB1) + (wave & 1) * 16384;
        else if constexpr (RBA == 128)
            reg = (wave < 4 ? sA0 : sA1) + (wave & 3) * 8192;
        else
            reg = (wave < 4 ? sB0 : sB1) + (wave & 3) * 8192;
        constexpr int ESZ = BF16OUT ? 2 : 4;
        constexpr int ROWB = 64 * ESZ;             // bytes per row of the wave's tile
        constexpr int CPR = ROWB / 16;             // 16-byte chunks per row: 8 or 16
        constexpr int PASS_ROWS = REG / ROWB;      // rows per pass: 128, 64 or 32
        constexpr int PASSES = 128 / PASS_ROWS;
        const int mbase = m0 + wm * 128, nbase = n0 + wn * 64;
        const bool full_cols = nbase + 64 <= g.N;
        const bool vec = full_cols && (g.ldc % (16 / ESZ) == 0) && (((uintptr_t)g.c & 15) == 0);
#pragma unroll
        for (int pass = 0; pass < PASSES; pass++) {
#pragma unroll
            for (int ii = 0; ii < 4 / PASSES; ii++) {
                const int i = pass * (4 / PASSES) + ii;
                const int m = ii * 32 + l32;  // row within the pass
#pragma unroll
                for (int j = 0; j < 2; j++)
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const float v0 = value(i, j, q, 0), v1 = value(i, j, q, 1);
                        const float v2 = value(i, j, q, 2), v3 = value(i, j, q, 3);
                        if constexpr (BF16OUT) {
                            const int c = 4 * j + q;  // 8-byte half h of 16-byte chunk c
                            const int off = m * ROWB + ((c ^ (m & (CPR - 1))) << 4) + 8 * h;
                            *reinterpret_cast<uint2 *>(&reg[off]) =
                                make_uint2(bf16x2(v0, v1), bf16x2(v2, v3));
                        } else {
                            const int c = 8 * j + 2 * q + h;
                            const int off = m * ROWB + ((c ^ (m & (CPR - 1))) << 4);
                            *reinterpret_cast<float4 *>(&reg[off]) = make_float4(v0, v1, v2, v3);
                        }
                    }
            }
            // read back row-contiguous: lane -> row lane / CPR (+ 64 / CPR per step), chunk lane % CPR
#pragma unroll
            for (int step = 0; step < PASS_ROWS * CPR / 64; step++) {
                const int m = step * (64 / CPR) + lane / CPR, c = lane % CPR;
                const uint4 t = *reinterpret_cast<const uint4 *>(&reg[m * ROWB + ((c ^ (m & (CPR - 1))) << 4)]);
                const int gm = mbase + pass * PASS_ROWS + m, gn = nbase + c * (16 / ESZ);
                if (gm >= g.M) continue;
                if (vec) {
                    // non-temporal: C is not read again by this kernel, and the lines should not
                    // linger dirty in the last-level cache for the next kernel to write back
                    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                    __builtin_nontemporal_store(
                        u32x4{t.x, t.y, t.z, t.w},
                        reinterpret_cast<u32x4 *>(reinterpret_cast<uint8_t *>(g.c) + ((int64_t)gm * g.ldc + gn) * ESZ));
                } else {
                    const uint32_t w4[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                    for (int e = 0; e < 16 / ESZ; e++) {
                        if (gn + e >= g.N) break;
                        if constexpr (BF16OUT)
                            reinterpret_cast<uint16_t *>(g.c)[(int64_t)gm * g.ldc + gn + e] =
                                (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                        else
                            reinterpret_cast<uint32_t *>(g.c)[(int64_t)gm * g.ldc + gn + e] = w4[e];
                    }
                }
            }
        }
    } else {
        const bool vec = (g.ldc % 4 == 0) && (((uintptr_t)g.c & (BF16OUT ? 7 : 15)) == 0);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int q = 0; q < 4; q++)
                    store_c4<BF16OUT>(g, m0 + wm * 128 + i * 32 + l32, n0 + wn * 64 + j * 32 + 8 * q + 4 * h,
                                      value(i, j, q, 0), value(i, j, q, 1), value(i, j, q, 2), value(i, j, q, 3), vec);
    }
}

}  // namespace pipe

// C = 0 for K == 0
template <bool BF16OUT>
__global__ void k_zero(void *c, int64_t ldc, int M, int N) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)M * N) return;
    const int64_t m = i / N, n = i % N;
    if (BF16OUT)
        reinterpret_cast<uint16_t *>(c)[m * ldc + n] = 0;
    else
        reinterpret_cast<float *>(c)[m * ldc + n] = 0.f;
}

template <int FA, int FB>
hipError_t launch_fmt(const GemmArgs &g, bool bf16, hipStream_t stream) {
    const dim3 grid((unsigned)(g.tiles_m * g.tiles_n)), block(NT);
    constexpr bool fp4 = FA == E2M1 && FB == E2M1;
    // pipelined kernels: K a whole number of scale slots (16 scale bytes =
    // 512 elements per row), code and scale row strides multiples of 16 bytes
    // (as the dense ones are then), 16-byte aligned code and dword-aligned
    // scale pointers, offsets in 32 bits
    const int64_t ldmax = g.lda > g.ldb ? g.lda : g.ldb, ldsmax = g.ldsa > g.ldsb ? g.ldsa : g.ldsb;
    const bool pipelined = g.K % 512 == 0 && ((uintptr_t)g.a % 16 == 0) && ((uintptr_t)g.b % 16 == 0) &&
                           ((uintptr_t)g.as % 4 == 0) && ((uintptr_t)g.bs % 4 == 0) &&
                           g.lda % 16 == 0 && g.ldb % 16 == 0 && g.ldsa % 16 == 0 && g.ldsb % 16 == 0 &&
                           (int64_t)BM * ldmax < ((int64_t)1 << 31) && (int64_t)BM * ldsmax < ((int64_t)1 << 31);
    if (g.kpa || g.kpb) {
        // K-panel operands: the pipelined kernels only, with 128-byte stage rows (E2M1 beside
        // E2M1, or FP8), and every panel offset in 31 bits
        constexpr int KE = fp4 ? 256 : 128;
        constexpr int RBA = FA == E2M1 ? KE / 2 : KE, RBB = FB == E2M1 ? KE / 2 : KE;
        const int64_t ntk = g.K / KE;
        if (!pipelined || (g.kpa && (RBA != 128 || ntk * g.kpa >= ((int64_t)1 << 31))) ||
            (g.kpb && (RBB != 128 || ntk * g.kpb >= ((int64_t)1 << 31))))
            return hipErrorInvalidValue;
    }
    if (pipelined) {
        const dim3 block(pipe::PNT);
        if constexpr (fp4) {
            if (bf16)
                hipLaunchKernelGGL((pipe::k_gemm_pipe<FA, FB, true, 0>), grid, block, 0, stream, g);
            else
                hipLaunchKernelGGL((pipe::k_gemm_pipe<FA, FB, false, 0>), grid, block, 0, stream, g);
        } else {
            if (bf16) {
                hipLaunchKernelGGL((pipe::k_gemm_pipe<FA, FB, true, 1>), grid, block, 0, stream, g);
                hipLaunchKernelGGL((pipe::k_gemm_pipe<FA, FB, true, 2>), grid, block, 0, stream, g);
            } else {
                hipLaunchKernelGGL((pipe::k_gemm_pipe<FA, FB, false, 1>), grid, block, 0, stream, g);
                hipLaunchKernelGGL((pipe::k_gemm_pipe<FA, FB, false, 2>), grid, block, 0, stream, g);
            }
        }
        return hipGetLastError();
    }
    if constexpr (fp4) {
        if (bf16)
            hipLaunchKernelGGL((k_gemm_fp4<true>), grid, block, 0, stream, g);
        else
            hipLaunchKernelGGL((k_gemm_fp4<false>), grid, block, 0, stream, g);
    } else {
        if (bf16) {
            hipLaunchKernelGGL((k_gemm_carrier<FA, FB, true, false>), grid, block, 0, stream, g);
            hipLaunchKernelGGL((k_gemm_carrier<FA, FB, true, true>), grid, block, 0, stream, g);
        } else {
            hipLaunchKernelGGL((k_gemm_carrier<FA, FB, false, false>), grid, block, 0, stream, g);
            hipLaunchKernelGGL((k_gemm_carrier<FA, FB, false, true>), grid, block, 0, stream, g);
        }
    }
    return hipGetLastError();
}

}  // namespace
}  // namespace mx
