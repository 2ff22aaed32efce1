// mx_gemm_e5m2_e2m1.hip -- MX GEMM kernels for A in E5M2 and B in E2M1
#include "mx_gemm_kernels.h"

namespace mx {
hipError_t launch_gemm_pair_1_2(const GemmArgs &g, bool bf16, hipStream_t s) { return launch_fmt<1, 2>(g, bf16, s); }
}  // namespace mx
