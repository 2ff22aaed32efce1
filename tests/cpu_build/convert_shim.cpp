// Host build of the HIP path's element conversion (precision_block_amax_amd/csrc/mx_convert.h)
// so the test suite can compare it exhaustively with the oracle without a GPU.
#include <stdint.h>
#include "mx_convert.h"

template <int F>
static void run_bf16(const uint16_t *b, const int32_t *e, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)mx::code_from_bf16<F>(b[i], e[i]);
}
template <int F>
static void run_f32(const float *y, const int32_t *e, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)mx::code_from_f32<F>(y[i], e[i]);
}

extern "C" {
int shim_code_from_bf16(const uint16_t *b, const int32_t *e, int64_t n, int fmt, uint8_t *out) {
    switch (fmt) {
    case 0: run_bf16<mx::E4M3>(b, e, n, out); return 0;
    case 1: run_bf16<mx::E5M2>(b, e, n, out); return 0;
    case 2: run_bf16<mx::E2M1>(b, e, n, out); return 0;
    }
    return -1;
}
int shim_code_from_f32(const float *y, const int32_t *e, int64_t n, int fmt, uint8_t *out) {
    switch (fmt) {
    case 0: run_f32<mx::E4M3>(y, e, n, out); return 0;
    case 1: run_f32<mx::E5M2>(y, e, n, out); return 0;
    case 2: run_f32<mx::E2M1>(y, e, n, out); return 0;
    }
    return -1;
}
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
