// mx_gemm.hip -- MX-scaled GEMM for gfx950: C[m, n] = sum_k A[m, k] * B[n, k],
// both operands MX-quantized with K contiguous (codes + one E8M0 scale per
// 32-element block), fp32 accumulation, fp32 or bf16 output.
//
// The linear-layer GEMMs (forward, activation gradient, weight gradient) of
// quantized training (FP4-training article on hzrcw.cc, section 02), which
// the Primus page identifies as the dominant training cost.
//
// Two kernels share one tiling (MFMA-bound; 2*M*N*K flops):
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
// binades, or which holds an E8M0 NaN (0xFF), is left to a second kernel with
// an exact per-block path: each 32-element block's partial sum of unscaled
// codes is scaled with ldexp and added in fp32 (separate kernels keep the
// VALU-side accumulation out of the fast kernel's register budget).
#include <type_traits>

#include "mx_internal.h"

namespace mx {
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

struct GemmArgs {
    const uint8_t *a, *as, *b, *bs;
    void *c;
    int64_t ldc;
    int M, N, K;
    int tiles_m, tiles_n;
};

// byte offset of 16-byte chunk `ch` of row `row` in a swizzled LDS tile
template <int RB>
__device__ __forceinline__ int swz(int row, int ch) {
    if constexpr (RB == 128) return row * 128 + ((ch ^ (row & 7)) << 4);
    else return row * 64 + ((ch ^ ((row >> 1) & 3)) << 4);  // 64-byte rows: two rows per 128 bytes
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

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
            ra[i] = off < rowA ? *reinterpret_cast<const uint4 *>(g.a + gr * rowA + off) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < NLB; i++) {
            const int id = tid + NT * i, row = id / CPRB, ch = id % CPRB;
            const int gr = min(n0 + row, g.N - 1);
            const int64_t off = (int64_t)kt * RBB + ch * 16;
            rb[i] = off < rowB ? *reinterpret_cast<const uint4 *>(g.b + gr * rowB + off) : make_uint4(0, 0, 0, 0);
        }
        // scales: thread t owns row t of the A and B tiles
        const int ga = min(m0 + tid, g.M - 1), gb = min(n0 + tid, g.N - 1);
        const int kb0 = kt * SB;
        if (scale_vec && kb0 + SB <= kblocks) {
            if constexpr (SB == 4) {
                rsa[0] = *reinterpret_cast<const uint32_t *>(g.as + (int64_t)ga * kblocks + kb0);
                rsb[0] = *reinterpret_cast<const uint32_t *>(g.bs + (int64_t)gb * kblocks + kb0);
            } else {
                const uint2 ta = *reinterpret_cast<const uint2 *>(g.as + (int64_t)ga * kblocks + kb0);
                const uint2 tb = *reinterpret_cast<const uint2 *>(g.bs + (int64_t)gb * kblocks + kb0);
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
                        va |= (uint32_t)g.as[(int64_t)ga * kblocks + kb] << (8 * t);
                        vb |= (uint32_t)g.bs[(int64_t)gb * kblocks + kb] << (8 * t);
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
    const bool scale_vec = (kblocks % SB == 0) && (((uintptr_t)g.as | (uintptr_t)g.bs) % SB == 0);

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

// the 8 codes of row `row`, elements [16s + 8h, 16s + 8h + 8) of the K tile
template <int F, int RB>
__device__ __forceinline__ void read_codes(const uint8_t *tile, int row, int s, int h, uint32_t &lo, uint32_t &hi) {
    if constexpr (F == E2M1) {
        const int byte = 8 * s + 4 * h;  // 4 bytes
        lo = *reinterpret_cast<const uint32_t *>(&tile[swz<RB>(row, byte >> 4) + (byte & 15)]);
        hi = 0;
    } else {
        const int byte = 16 * s + 8 * h;  // 8 bytes
        const uint2 t = *reinterpret_cast<const uint2 *>(&tile[swz<RB>(row, byte >> 4) + (byte & 15)]);
        lo = t.x;
        hi = t.y;
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
    const bool scale_vec = (kblocks % SB == 0) && (((uintptr_t)g.as | (uintptr_t)g.bs) % SB == 0);

    // reference scales R = max over the row's blocks; the tile is "wide" if a
    // row's scales spread over more than kSpreadMax binades or hold 0xFF
    bool wide;
    {
        const int ga = min(m0 + tid, g.M - 1), gb = min(n0 + tid, g.N - 1);
        int amax = 0, amin = 255, bmax = 0, bmin = 255;
        const uint8_t *pa = g.as + (int64_t)ga * kblocks, *pb = g.bs + (int64_t)gb * kblocks;
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
                        const float v = __builtin_amdgcn_ldexpf(p[r], sa_r[r] + sb - 254);
                        acc[i][j][r] += (sa_r[r] == 255 || sb == 255) ? __builtin_nanf("") : v;
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
    if constexpr (FA == E2M1 && FB == E2M1) {
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

template <int FA>
hipError_t launch_fa(const GemmArgs &g, int fb, bool bf16, hipStream_t stream) {
    switch (fb) {
    case E4M3: return launch_fmt<FA, E4M3>(g, bf16, stream);
    case E5M2: return launch_fmt<FA, E5M2>(g, bf16, stream);
    default: return launch_fmt<FA, E2M1>(g, bf16, stream);
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t *a, const uint8_t *as, int fa, const uint8_t *b, const uint8_t *bs, int fb,
                       int64_t M, int64_t N, int64_t K, void *c, bool bf16_out, int64_t ldc, hipStream_t stream) {
    if (K == 0) {
        const int64_t n = M * N;
        const dim3 grid((unsigned)((n + 255) / 256));
        if (bf16_out)
            hipLaunchKernelGGL((k_zero<true>), grid, dim3(256), 0, stream, c, ldc, (int)M, (int)N);
        else
            hipLaunchKernelGGL((k_zero<false>), grid, dim3(256), 0, stream, c, ldc, (int)M, (int)N);
        return hipGetLastError();
    }
    GemmArgs g;
    g.a = a; g.as = as; g.b = b; g.bs = bs; g.c = c; g.ldc = ldc;
    g.M = (int)M; g.N = (int)N; g.K = (int)K;
    g.tiles_m = (int)((M + BM - 1) / BM);
    g.tiles_n = (int)((N + BN - 1) / BN);
    switch (fa) {
    case E4M3: return launch_fa<E4M3>(g, fb, bf16_out, stream);
    case E5M2: return launch_fa<E5M2>(g, fb, bf16_out, stream);
    default: return launch_fa<E2M1>(g, fb, bf16_out, stream);
    }
}

}  // namespace mx
