// mx_gemm_e4m3_e5m2.hip -- MX GEMM kernels for A in E4M3 and B in E5M2
#include "mx_gemm_kernels.h"

namespace mx {
hipError_t launch_gemm_pair_0_1(const GemmArgs &g, bool bf16, hipStream_t s) { return launch_fmt<0, 1>(g, bf16, s); }
}  // namespace mx
