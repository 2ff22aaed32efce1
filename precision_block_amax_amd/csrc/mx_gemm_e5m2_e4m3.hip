// mx_gemm_e5m2_e4m3.hip -- MX GEMM kernels for A in E5M2 and B in E4M3
#include "mx_gemm_kernels.h"

namespace mx {
hipError_t launch_gemm_pair_1_0(const GemmArgs &g, bool bf16, hipStream_t s) { return launch_fmt<1, 0>(g, bf16, s); }
}  // namespace mx
