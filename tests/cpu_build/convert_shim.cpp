// Host build of the kernels' E8M0 scale-exponent functions
// (precision_block_amax_amd/csrc/mx_convert.h) so the test suite can compare
// them exhaustively with the oracle without a GPU.
#include <stdint.h>
#include "mx_convert.h"

extern "C" {
int shim_scale_exp_bf16(const uint16_t *a, int64_t n, int fmt, int32_t *out) {
    for (int64_t i = 0; i < n; i++) {
        uint32_t m = a[i] & 0x7FFFu;
        out[i] = fmt == 0 ? mx::scale_exp_bf16<mx::E4M3>(m) : fmt == 1 ? mx::scale_exp_bf16<mx::E5M2>(m)
                                                                          : mx::scale_exp_bf16<mx::E2M1>(m);
    }
    return 0;
}
int shim_scale_exp_f32(const uint32_t *a, int64_t n, int fmt, int32_t *out) {
    for (int64_t i = 0; i < n; i++) {
        uint32_t m = a[i] & 0x7FFFFFFFu;
        out[i] = fmt == 0 ? mx::scale_exp_f32<mx::E4M3>(m) : fmt == 1 ? mx::scale_exp_f32<mx::E5M2>(m)
                                                                         : mx::scale_exp_f32<mx::E2M1>(m);
    }
    return 0;
}
}
