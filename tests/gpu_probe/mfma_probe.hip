// mfma_probe.hip -- test-only probes of single gfx950 matrix instructions.
//
// Not part of libmx: the test suite builds this into libmfma_probe.so to show,
// on the device, the arithmetic facts the GEMM's design rests on:
//   - the block-scaled FP8 instruction (V_MFMA_SCALE_F32_32X32X64_F8F6F4 with
//     E4M3 operands) does not sum a 32-element block exactly in fp32, so MX
//     GEMMs with an FP8 operand cannot meet an fp32-accumulation tolerance on
//     it and run through an exact bf16 carrier instead;
//   - the same instruction on E2M1 operands, and the bf16 instruction
//     V_MFMA_F32_32X32X16_BF16, sum their products exactly and round once.
// Each probe runs one wave, one instruction, on 32 x K operands given row-major
// with K contiguous (A: M rows, B: N rows), and writes C[32 x 32] row-major
// with C[m][n] = sum_k A[m][k] * B[n][k] (times the block scales).
//
// Operand layout of the 32x32x64 scaled instruction (lane l, h = l / 32):
// lane l supplies row l % 32; for FP8 its 32 bytes are K[16h, 16h + 16) then
// K[32 + 16h, 32 + 16h + 16); for E2M1 its 16 bytes are K[32h, 32h + 32).
// Lanes of group h supply the E8M0 scale of K block h (byte 0 of the scale
// register here).  Output: lane l holds column l % 32, rows
// 8 (r / 4) + 4 h + r % 4 for r = 0 .. 15.  The bf16 32x32x16 instruction:
// lane l supplies row l % 32, K[8h, 8h + 8).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {

__device__ void store_c(float *c, const v16f &acc) {
    const int l = threadIdx.x, h = l >> 5;
    for (int r = 0; r < 16; r++) c[(8 * (r >> 2) + 4 * h + (r & 3)) * 32 + (l & 31)] = acc[r];
}

// FP4 = true: E2M1 codes, two per byte (element 2i in the low nibble), K = 64
template <bool FP4>
__global__ void k_scaled(const uint8_t *a, const uint8_t *b, const uint8_t *sa, const uint8_t *sb, float *c) {
    const int l = threadIdx.x, row = l & 31, h = l >> 5;
    int wa[8] = {0, 0, 0, 0, 0, 0, 0, 0}, wb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (FP4) {
        for (int q = 0; q < 4; q++) {  // bytes [16h, 16h + 16) of the 32-byte row
            wa[q] = *reinterpret_cast<const int *>(a + row * 32 + 16 * h + 4 * q);
            wb[q] = *reinterpret_cast<const int *>(b + row * 32 + 16 * h + 4 * q);
        }
    } else {
        for (int q = 0; q < 4; q++) {
            wa[q] = *reinterpret_cast<const int *>(a + row * 64 + 16 * h + 4 * q);
            wa[4 + q] = *reinterpret_cast<const int *>(a + row * 64 + 32 + 16 * h + 4 * q);
            wb[q] = *reinterpret_cast<const int *>(b + row * 64 + 16 * h + 4 * q);
            wb[4 + q] = *reinterpret_cast<const int *>(b + row * 64 + 32 + 16 * h + 4 * q);
        }
    }
    const v8i va = {wa[0], wa[1], wa[2], wa[3], wa[4], wa[5], wa[6], wa[7]};
    const v8i vb = {wb[0], wb[1], wb[2], wb[3], wb[4], wb[5], wb[6], wb[7]};
    const int scale_a = sa[row * 2 + h], scale_b = sb[row * 2 + h];
    v16f acc;
    for (int r = 0; r < 16; r++) acc[r] = 0.f;
    constexpr int FMT = FP4 ? 4 : 0;  // cbsz / blgp: 0 = E4M3, 4 = E2M1
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, FMT, FMT, 0, scale_a, 0, scale_b);
    store_c(c, acc);
}

__global__ void k_bf16(const uint16_t *a, const uint16_t *b, float *c) {
    const int l = threadIdx.x, row = l & 31, h = l >> 5;
    v8bf va, vb;
    for (int i = 0; i < 8; i++) {
        va[i] = __builtin_bit_cast(__bf16, a[row * 16 + 8 * h + i]);
        vb[i] = __builtin_bit_cast(__bf16, b[row * 16 + 8 * h + i]);
    }
    v16f acc;
    for (int r = 0; r < 16; r++) acc[r] = 0.f;
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc, 0, 0, 0);
    store_c(c, acc);
}

int finish() {
    if (hipGetLastError() != hipSuccess) return 1;
    return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}

}  // namespace

extern "C" {

// A, B: 32 x 64 E4M3 codes (row-major); sa, sb: 32 x 2 E8M0 scales; c: 32 x 32 fp32.
// Device pointers.  Returns 0, or 1 on a HIP error.  Synchronizes.
int probe_mfma_scale_e4m3(const uint8_t *a, const uint8_t *b, const uint8_t *sa, const uint8_t *sb, float *c) {
    hipLaunchKernelGGL(k_scaled<false>, dim3(1), dim3(64), 0, 0, a, b, sa, sb, c);
    return finish();
}

// A, B: 32 x 64 E2M1 codes packed two per byte (32 x 32 bytes); scales and c as above.
int probe_mfma_scale_e2m1(const uint8_t *a, const uint8_t *b, const uint8_t *sa, const uint8_t *sb, float *c) {
    hipLaunchKernelGGL(k_scaled<true>, dim3(1), dim3(64), 0, 0, a, b, sa, sb, c);
    return finish();
}

// A, B: 32 x 16 bf16 (row-major bit patterns); c: 32 x 32 fp32.
int probe_mfma_bf16(const uint16_t *a, const uint16_t *b, float *c) {
    hipLaunchKernelGGL(k_bf16, dim3(1), dim3(64), 0, 0, a, b, c);
    return finish();
}

}  // extern "C"
