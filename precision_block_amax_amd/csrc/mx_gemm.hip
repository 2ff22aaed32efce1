// mx_gemm.hip -- MX-scaled GEMM for gfx950: C[m, n] = sum_k A[m, k] * B[n, k],
// both operands MX-quantized with K contiguous (codes + one E8M0 scale per
// 32-element block), fp32 accumulation, fp32 or bf16 output.
//
// The linear-layer GEMMs (forward, activation gradient, weight gradient) of
// quantized training (FP4-training article on hzrcw.cc, section 02), which
// the Primus page identifies as the dominant training cost.
//
// Design (MFMA-bound; 2*M*N*K flops):
//   - V_MFMA_SCALE_F32_32X32X64_F8F6F4 (K = 64 per instruction): lane l
//     serves row l % 32 of A (column of B); its half h = l / 32 supplies the
//     E8M0 byte of K block h, and the matrix core applies both scales, so
//     there is no dequantization pass.  Operand bytes per lane (measured on
//     gfx950): FP4 -- 16 bytes = K[32h, 32h+32), one whole block; FP8 -- 32
//     bytes = K[16h, 16h+16) followed by K[32+16h, 32+16h+16), i.e. 16-byte
//     chunks h and 2+h of the 64-byte K step.  FP8 (E4M3 / E5M2) and FP4
//     (E2M1) operands mix freely.
//   - Workgroup tile 256 x 256, four waves of 128 x 128 (4 x 4 MFMA tiles,
//     256 fp32 accumulators per lane).  K tile: 128 bytes of codes per row
//     (128 FP8 or 256 FP4 elements).
//   - Operand tiles are double-buffered in LDS (2 x 64 KiB) with the 16-byte
//     chunks of each row XOR-swizzled by the row index, so the 32 lanes that
//     read the same K chunk of 32 consecutive rows hit distinct banks.  One
//     barrier per K tile; the next tile's global loads are in flight while
//     the current tile is multiplied.
//   - Scales of a K tile (4 or 8 bytes per row) are staged in LDS beside the
//     codes; a lane selects its block's byte with the instruction's op_sel.
//   - Tile order: workgroups are dealt round-robin to the 8 XCDs, so each XCD
//     gets a contiguous run of tiles, ordered in groups of 8 tile rows, to keep
//     shared A rows and B columns in that XCD's L2.
//   - M and N tails: loads clamp to the last valid row and stores are masked;
//     the K tail is zero-filled (code 0, scale byte 0).
#include <type_traits>

#include "mx_internal.h"

namespace mx {
namespace {

// compile-time loop: f(std::integral_constant<int, I>) for I in [I0, N)
template <int I, int N, class Fn>
__device__ __forceinline__ void static_for(Fn &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, NT = 256;

// matrix-core format selector (cbsz / blgp)
template <int F> struct MfmaFmt;
template <> struct MfmaFmt<E4M3> { static constexpr int v = 0; };
template <> struct MfmaFmt<E5M2> { static constexpr int v = 1; };
template <> struct MfmaFmt<E2M1> { static constexpr int v = 4; };

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
    if (RB == 128) return row * 128 + ((ch ^ (row & 7)) << 4);
    return row * 64 + ((ch ^ ((row >> 1) & 3)) << 4);  // 64-byte rows: two rows per 128 bytes
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;  // quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int FA, int FB, bool BF16OUT>
__global__ __launch_bounds__(NT, 1) void k_gemm(GemmArgs g) {
    constexpr bool A4 = FA == E2M1, B4 = FB == E2M1;
    constexpr int BK = (A4 && B4) ? 256 : 128;  // K elements per tile
    constexpr int RBA = A4 ? BK / 2 : BK;       // LDS row bytes
    constexpr int RBB = B4 ? BK / 2 : BK;
    constexpr int SB = BK / 32;                 // scale bytes per row per tile
    constexpr int STEPS = BK / 64;              // MFMAs along K per tile
    constexpr int CPRA = RBA / 16, CPRB = RBB / 16;
    constexpr int NLA = BM * CPRA / NT, NLB = BN * CPRB / NT;

    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * RBA];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * RBB];
    __shared__ __attribute__((aligned(16))) uint8_t sAs[2][BM * SB];
    __shared__ __attribute__((aligned(16))) uint8_t sBs[2][BN * SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;

    // XCD-aware tile order
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
    const int tm = first_m + in_grp % gsz;
    const int tn = in_grp / gsz;
    const int m0 = tm * BM, n0 = tn * BN;

    const int K = g.K;
    const int64_t rowA = A4 ? K / 2 : K, rowB = B4 ? K / 2 : K;
    const int kblocks = K / 32;
    const int ntk = (K + BK - 1) / BK;
    const bool scale_vec = (kblocks % SB == 0) && (((uintptr_t)g.as | (uintptr_t)g.bs) % SB == 0);

    uint4 ra[NLA], rb[NLB];
    uint32_t rsa[SB / 4], rsb[SB / 4];

    auto load_tile = [&](int kt) {
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
    };

    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NLA; i++) {
            const int id = tid + NT * i, row = id / CPRA, ch = id % CPRA;
            *reinterpret_cast<uint4 *>(&sA[buf][swz<RBA>(row, ch)]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < NLB; i++) {
            const int id = tid + NT * i, row = id / CPRB, ch = id % CPRB;
            *reinterpret_cast<uint4 *>(&sB[buf][swz<RBB>(row, ch)]) = rb[i];
        }
#pragma unroll
        for (int q = 0; q < SB / 4; q++) {
            reinterpret_cast<uint32_t *>(&sAs[buf][tid * SB])[q] = rsa[q];
            reinterpret_cast<uint32_t *>(&sBs[buf][tid * SB])[q] = rsb[q];
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    auto compute = [&](int buf) {
        // per-lane scale words: byte 2s of (word >> 8h) is block 2s + h of this tile
        uint32_t sa[4][SB / 4], sbw[4][SB / 4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int ra_ = wm * 128 + i * 32 + l32, rb_ = wn * 128 + i * 32 + l32;
#pragma unroll
            for (int q = 0; q < SB / 4; q++) {
                sa[i][q] = reinterpret_cast<const uint32_t *>(&sAs[buf][ra_ * SB])[q] >> (8 * h);
                sbw[i][q] = reinterpret_cast<const uint32_t *>(&sBs[buf][rb_ * SB])[q] >> (8 * h);
            }
        }
        static_for<0, STEPS>([&](auto step) {
            constexpr int s = decltype(step)::value;
            v8i fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int row = wm * 128 + i * 32 + l32;
                if constexpr (A4) {
                    const uint4 t = *reinterpret_cast<const uint4 *>(&sA[buf][swz<RBA>(row, 2 * s + h)]);
                    fa[i] = v8i{(int)t.x, (int)t.y, (int)t.z, (int)t.w, 0, 0, 0, 0};
                } else {
                    const uint4 t0 = *reinterpret_cast<const uint4 *>(&sA[buf][swz<RBA>(row, 4 * s + h)]);
                    const uint4 t1 = *reinterpret_cast<const uint4 *>(&sA[buf][swz<RBA>(row, 4 * s + 2 + h)]);
                    fa[i] = v8i{(int)t0.x, (int)t0.y, (int)t0.z, (int)t0.w, (int)t1.x, (int)t1.y, (int)t1.z, (int)t1.w};
                }
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int row = wn * 128 + j * 32 + l32;
                if constexpr (B4) {
                    const uint4 t = *reinterpret_cast<const uint4 *>(&sB[buf][swz<RBB>(row, 2 * s + h)]);
                    fb[j] = v8i{(int)t.x, (int)t.y, (int)t.z, (int)t.w, 0, 0, 0, 0};
                } else {
                    const uint4 t0 = *reinterpret_cast<const uint4 *>(&sB[buf][swz<RBB>(row, 4 * s + h)]);
                    const uint4 t1 = *reinterpret_cast<const uint4 *>(&sB[buf][swz<RBB>(row, 4 * s + 2 + h)]);
                    fb[j] = v8i{(int)t0.x, (int)t0.y, (int)t0.z, (int)t0.w, (int)t1.x, (int)t1.y, (int)t1.z, (int)t1.w};
                }
            }
            constexpr int q = (2 * s) / 4;        // scale word holding blocks 2s, 2s+1
            constexpr int sel = (2 * s) % 4;      // its byte, after the >> 8h above
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[i], fb[j], acc[i][j], MfmaFmt<FA>::v, MfmaFmt<FB>::v, sel, (int)sa[i][q], sel,
                        (int)sbw[j][q]);
        });
    };

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < ntk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < ntk) load_tile(kt + 1);
        compute(cur);
        if (kt + 1 < ntk) store_tile(cur ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds column n = l32 and rows 8(r/4) + 4h + r%4 of each 32 x 32 tile
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int n = n0 + wn * 128 + j * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < g.M && n < g.N) {
                    if (BF16OUT)
                        reinterpret_cast<uint16_t *>(g.c)[(int64_t)m * g.ldc + n] = (uint16_t)bf16_rne(acc[i][j][r]);
                    else
                        reinterpret_cast<float *>(g.c)[(int64_t)m * g.ldc + n] = acc[i][j][r];
                }
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
    if (bf16)
        hipLaunchKernelGGL((k_gemm<FA, FB, true>), grid, block, 0, stream, g);
    else
        hipLaunchKernelGGL((k_gemm<FA, FB, false>), grid, block, 0, stream, g);
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

hipError_t launch_gemm(const uint8_t *a, const uint8_t *as, int fa, const uint8_t *b, const uint8_t *bs,
                       int fb, int64_t M, int64_t N, int64_t K, void *c, bool bf16_out, int64_t ldc,
                       hipStream_t stream) {
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
