// mx_gemm.hip -- dispatch of mx_gemm to the kernels of mx_gemm_kernels.h.
// Each operand-format pair is instantiated in its own translation unit
// (mx_gemm_<fa>_<fb>.hip) so the library builds in parallel.
#include "mx_gemm_kernels.h"

namespace mx {

#define MX_PAIR(fa, fb) hipError_t launch_gemm_pair_##fa##_##fb(const GemmArgs &g, bool bf16, hipStream_t s);
MX_PAIR(0, 0) MX_PAIR(0, 1) MX_PAIR(0, 2)
MX_PAIR(1, 0) MX_PAIR(1, 1) MX_PAIR(1, 2)
MX_PAIR(2, 0) MX_PAIR(2, 1) MX_PAIR(2, 2)
#undef MX_PAIR

hipError_t launch_gemm(const uint8_t *a, int64_t lda, const uint8_t *as, int64_t ldsa, int fa, const uint8_t *b,
                       int64_t ldb, const uint8_t *bs, int64_t ldsb, int fb, int64_t M, int64_t N, int64_t K, void *c,
                       bool bf16_out, int64_t ldc, hipStream_t stream, int64_t kpa, int64_t kpb) {
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
    g.lda = lda; g.ldsa = ldsa; g.ldb = ldb; g.ldsb = ldsb;
    g.kpa = kpa; g.kpb = kpb;
    g.M = (int)M; g.N = (int)N; g.K = (int)K;
    g.tiles_m = (int)((M + BM - 1) / BM);
    g.tiles_n = (int)((N + BN - 1) / BN);
    switch (fa * 3 + fb) {
    case 0: return launch_gemm_pair_0_0(g, bf16_out, stream);
    case 1: return launch_gemm_pair_0_1(g, bf16_out, stream);
    case 2: return launch_gemm_pair_0_2(g, bf16_out, stream);
    case 3: return launch_gemm_pair_1_0(g, bf16_out, stream);
    case 4: return launch_gemm_pair_1_1(g, bf16_out, stream);
    case 5: return launch_gemm_pair_1_2(g, bf16_out, stream);
    case 6: return launch_gemm_pair_2_0(g, bf16_out, stream);
    case 7: return launch_gemm_pair_2_1(g, bf16_out, stream);
    default: return launch_gemm_pair_2_2(g, bf16_out, stream);
    }
}

}  // namespace mx
