// mx_gemm_e2m1_e4m3.hip -- MX GEMM kernels for A in E2M1 and B in E4M3
#include "mx_gemm_kernels.h"

namespace mx {
hipError_t launch_gemm_pair_2_0(const GemmArgs &g, bool bf16, hipStream_t s) { return launch_fmt<2, 0>(g, bf16, s); }
}  // namespace mx
