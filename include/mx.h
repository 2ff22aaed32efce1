/*
 * mx.h -- C ABI of libmx: OCP-MX micro-scaling quantization, the fixed-sign
 * 32-point block-Hadamard rotation, and the MX-scaled GEMM, for AMD gfx950
 * (Instinct MI355X).
 *
 * What the calls compute, and where it is stated:
 *   - MX micro-scaling (FP4-training article on hzrcw.cc, section 02: the tensor
 *     is cut into small blocks, each with its own dynamic scaling exponent;
 *     MXFP4 is an OCP open format, section 04).  Block size 32 along the
 *     reduction dimension (MindSpeed-LLM FSDP2 quantization page: recipe
 *     dynamic_MX-1-1-32 and --model.quant_block_size 32).
 *   - Element formats E4M3 and E5M2 (Lumen page, section 1: E4M3 for
 *     precision, E5M2 for range) and E2M1 (MXFP4), OCP encodings: E4M3 "FN"
 *     (bias 7, max 448, no infinities), E5M2 (bias 15, max normal 57344),
 *     E2M1 (bias 1, max 6).  Shared scale: one E8M0 byte per block,
 *       S = clamp(floor(log2 amax) - emax, -127, 127) + 127,
 *     emax = 8 (E4M3), 15 (E5M2), 2 (E2M1); elements are v * 2^-(S-127),
 *     rounded to nearest (ties to even) and saturated to +-max normal.
 *   - The deterministic fixed-sign Hadamard rotation on the weight-gradient
 *     path (FP4-training article, section 02: one fixed orthogonal transform
 *     in place of random rotations), applied along tokens before the FP4
 *     quantization of both weight-gradient operands.
 *   - The quantized GEMMs of a linear layer (FP4-training article, section
 *     02: forward, activation-gradient and weight-gradient GEMMs), which the
 *     Primus page names as the dominant training cost (GEMM tuning section).
 *
 * Conventions shared by every call:
 *   - All data pointers are DEVICE pointers, allocated and freed by the
 *     caller.  The library allocates nothing and keeps no per-call state.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default (null)
 *     stream.  Calls are asynchronous on that stream and never synchronize.
 *   - Inputs are read only.  Outputs are overwritten completely (no
 *     accumulation).  Inputs and outputs must not overlap.
 *   - bf16 inputs are row-major with a leading dimension `ldx` (elements
 *     between the starts of consecutive rows, ldx >= cols).
 *   - Outputs are dense row-major (the _panels calls and pair modes write
 *     their codes in the K-panel layout described before them instead):
 *       FP8 codes   : one byte per element;
 *       E2M1 codes  : two elements per byte, element 2i in bits 3:0 and
 *                     element 2i+1 in bits 7:4;
 *       scales      : one E8M0 byte per 32-element block.
 *   - A block that holds an Inf or NaN gets scale 0xFF (E8M0 NaN) and all
 *     element codes 0.  An all-zero block gets scale 0x00.  The sign of zero
 *     is kept (-0 -> 0x80 for FP8, 0x8 for E2M1).
 *   - A size of 0 is a valid empty call: nothing is read or written (except
 *     mx_gemm with K == 0, which writes C = 0), and pointers may be NULL.
 *
 * Errors (no call throws, no call aborts):
 *   MX_ERR_INVALID_ARG  bad argument, detected on the host before any HIP
 *                       call: NULL pointer with a non-empty size, negative
 *                       size, a blocked dimension not a multiple of 32,
 *                       ldx < cols, ldc < N, unknown enum value, or
 *                       operand and output buffers that overlap.
 *   MX_ERR_UNSUPPORTED  the current device is not gfx950, or an index range
 *                       exceeds what the kernels address (more than 2^31
 *                       blocks or rows in one call).
 *   MX_ERR_HIP          a HIP runtime call or kernel launch failed.
 *   Faults inside a kernel surface at the caller's next synchronization.
 */
#ifndef MX_H
#define MX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MX_OK = 0,
    MX_ERR_INVALID_ARG = 1,
    MX_ERR_UNSUPPORTED = 2,
    MX_ERR_HIP = 3
} mx_status_t;

typedef enum {
    MX_E4M3 = 0, /* FP8 1-4-3, bias 7, max 448       */
    MX_E5M2 = 1, /* FP8 1-5-2, bias 15, max 57344    */
    MX_E2M1 = 2  /* FP4 1-2-1, bias 1, max 6, packed */
} mx_format_t;

typedef enum {
    MX_OUT_F32 = 0, /* fp32 output                          */
    MX_OUT_BF16 = 1 /* bf16 output, fp32 result rounded RNE */
} mx_out_t;

/*
 * mx_quantize -- row mode.  Block b of row r is x[r, 32b .. 32b+31].
 *   x_bf16  [rows x ldx] bf16, reads the first `cols` of each row
 *   cols    multiple of 32
 *   codes   [rows x cols] bytes (E4M3/E5M2) or [rows x cols/2] (E2M1)
 *   scales  [rows x cols/32] E8M0 bytes
 * This is the Fprop operand quantizer (activations and weights stored with
 * the reduction dimension contiguous) and the Dgrad quantizer of the output
 * gradient.
 * Defined by: FP4-training article on hzrcw.cc, section 02 (MX blocks, each
 * with its own dynamic power-of-two exponent, on the forward and
 * activation-gradient GEMM operands); MindSpeed-LLM FSDP2 page, section
 * "三步启用 MXFP8 低精度训练" (block size 32 along the reduction dimension);
 * Lumen page, section 1 (the E4M3 and E5M2 element formats).
 */
mx_status_t mx_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                        mx_format_t fmt, void *codes, void *scales, void *stream);

/*
 * mx_quantize_transpose -- transposed mode.  Block b of column c is
 * x[32b .. 32b+31, c]; it becomes block b of output row c, so the output is
 * the MX form of x^T with `rows` as its contiguous (reduction) dimension.
 *   rows    multiple of 32
 *   codes   [cols x rows] bytes (E4M3/E5M2) or [cols x rows/2] (E2M1)
 *   scales  [cols x rows/32]
 * Used for operands whose reduction dimension is strided in storage: the
 * weight in Dgrad (reduction over N_out) and, without rotation, the two
 * weight-gradient operands (reduction over tokens).
 * Defined by: FP4-training article on hzrcw.cc, section 02 (the
 * activation-gradient and weight-gradient GEMMs quantize their operands
 * along the GEMM's own reduction dimension), with the block and formats of
 * mx_quantize.
 */
mx_status_t mx_quantize_transpose(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                                  mx_format_t fmt, void *codes, void *scales, void *stream);

/*
 * mx_hadamard32_quantize -- transposed mode after the fixed-sign block
 * rotation.  For each column c and each 32-row block b, with
 * x_i = x[32b + i, c] widened to fp32:
 *     x_i <- -x_i  where bit i of sign_mask is set,
 *     five butterfly stages h = 1, 2, 4, 8, 16, each replacing
 *     (x_j, x_{j+h}) by (x_j + x_{j+h}, x_j - x_{j+h}) for every j with
 *     (j & h) == 0, one fp32 rounding per operation,
 *     y_i = x_i * c with c = 0x3E3504F3 = RN_fp32(1/sqrt(32)),
 * i.e. y = c * H32 * diag(s) * x with H32 the Sylvester-Hadamard matrix.
 * y (fp32, no bf16 rounding) is then quantized as block b of output row c,
 * with the same output layout as mx_quantize_transpose.  Rotation blocks
 * coincide with the MX blocks.  sign_mask = 0 is the plain Sylvester
 * rotation.  Results are bit-identical for every launch configuration.
 * Defined by: FP4-training article on hzrcw.cc, section 02 (one fixed,
 * deterministic Hadamard rotation of both weight-gradient operands along
 * tokens before the FP4 quantization, in place of random rotations).  The
 * sign vector, stage order, constant and fp32 arithmetic are the readings
 * written out above; the page gives the transform only in words.
 */
mx_status_t mx_hadamard32_quantize(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                                   uint32_t sign_mask, mx_format_t fmt, void *codes, void *scales,
                                   void *stream);

/*
 * mx_quantize_transpose_sr -- mx_quantize_transpose (rotate = 0) or
 * mx_hadamard32_quantize (rotate = 1, with sign_mask) with stochastic instead
 * of nearest rounding of the elements; same scales, same layout.  Stochastic
 * rounding is the randomised cast that the FP4-training article on hzrcw.cc
 * (section 01) names as the common remedy for FP4 training, against which it
 * argues for the deterministic rotation; it is here for that comparison.
 * Each element q = y * 2^-e (y the block value after the optional rotation,
 * e the block's scale exponent) lies between grid neighbours lo <= |q| < hi
 * and rounds up iff its 32-bit random word r < floor(2^32 (|q|-lo)/(hi-lo)),
 * so the up-probability is the fractional position to 32 bits; magnitudes
 * at or above the largest normal saturate; signs are kept.  Random words:
 * element t of output row c is element i = c * rows + t of the Philox4x32-10
 * stream (Salmon, Moraes, Dror, Shaw, SC 2011): word i mod 4 of the block at
 * counter (i / 4 low word, i / 4 high word, 0, 0) and key (seed low word,
 * seed high word).  The result depends only on x and seed, not on the launch
 * configuration.
 *   rotate  0 or 1
 * Sizes, layout, ownership and errors as mx_quantize_transpose.
 */
mx_status_t mx_quantize_transpose_sr(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx, int rotate,
                                     uint32_t sign_mask, uint64_t seed, mx_format_t fmt, void *codes, void *scales,
                                     void *stream);

/*
 * mx_quantize_dual -- the row form and the transposed form of x from one
 * read of x: codes_row / scales_row exactly as mx_quantize(x, fmt_row), and
 * codes_t / scales_t exactly as mx_quantize_transpose(x, fmt_t) (rotate = 0)
 * or mx_hadamard32_quantize(x, sign_mask, fmt_t) (rotate = 1).
 *   rows, cols  both multiples of 32
 *   rotate      0 or 1
 * A linear layer needs both forms of its activations, output gradients and
 * weights: the row form for Fprop and Dgrad, the transposed (for the
 * gradients, rotated) form for Dgrad's weight and for the weight gradient
 * (FP4-training article on hzrcw.cc, section 02).  The four output buffers
 * must not overlap each other or x.
 */
mx_status_t mx_quantize_dual(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                             mx_format_t fmt_row, void *codes_row, void *scales_row,
                             mx_format_t fmt_t, int rotate, uint32_t sign_mask, void *codes_t,
                             void *scales_t, void *stream);

typedef enum {
    MX_PAIR_ROW = 0,              /* as mx_quantize                               */
    MX_PAIR_TRANSPOSE = 1,        /* as mx_quantize_transpose                     */
    MX_PAIR_HADAMARD = 2,         /* as mx_hadamard32_quantize (sign_mask)        */
    MX_PAIR_TRANSPOSE_PANELS = 3, /* as mx_quantize_transpose_panels              */
    MX_PAIR_HADAMARD_PANELS = 4   /* as mx_hadamard32_quantize_panels (sign_mask) */
} mx_pair_mode_t;

/*
 * mx_quantize_pair -- the two operands of one GEMM in one launch.  x0 (rows0
 * x cols0, leading dimension ldx0) goes to codes0 / scales0 and x1 to codes1
 * / scales1, each exactly as the single call of `mode` would quantize it:
 * same format `fmt`, the same sign_mask for the rotated modes (ignored
 * otherwise), and per tensor the sizes, layouts, rules and errors of that
 * call.  The GEMMs of a linear layer take both operands in the same form
 * (FP4-training article on hzrcw.cc, section 02: Fprop X and W in row mode,
 * Wgrad dY and X rotated along tokens).  One launch for both saves one
 * launch's start-up and drain.  On MI355X that is 4-6% of the time for
 * the Llama-3.1-8B operand pairs.  Where the two need different
 * kernel variants (a strided or unaligned tensor), the call runs the two
 * single quantizations one after the other on `stream`; an empty tensor is
 * skipped.  Neither tensor's outputs may overlap the other tensor's input
 * or outputs (the two inputs may overlap: they are only read).
 */
mx_status_t mx_quantize_pair(mx_pair_mode_t mode, mx_format_t fmt, uint32_t sign_mask,
                             const void *x0, int64_t rows0, int64_t cols0, int64_t ldx0, void *codes0,
                             void *scales0, const void *x1, int64_t rows1, int64_t cols1, int64_t ldx1,
                             void *codes1, void *scales1, void *stream);

/*
 * mx_gemm -- C[m, n] = sum_k A[m, k] * B[n, k] over two MX operands, both
 * with the reduction dimension K contiguous ("TN"):
 *   a_codes [M x K] (FP8) or [M x K/2] (E2M1), a_scales [M x K/32]
 *   b_codes [N x K] (FP8) or [N x K/2] (E2M1), b_scales [N x K/32]
 *   A[m, k] = decode(code) * 2^(S - 127), same for B
 *   K       multiple of 32
 *   c       [M x ldc] fp32 or bf16 (per `out`), ldc >= N
 * E2M1 x E2M1 products are formed by the gfx950 block-scaled matrix
 * instruction (64 elements of K per step, exact), pairs with an FP8 operand
 * by the bf16 matrix instruction on codes converted exactly to bf16 against
 * a per-row reference scale; partial sums are accumulated in fp32, so
 * |C - sum| <= 1e-5 * sum |A[m, k] * B[n, k]|.  Fprop: A = X, B = W.
 * Dgrad: A = dY, B = W^T (from mx_quantize_transpose).  Wgrad: A = dY^T,
 * B = X^T (both from mx_hadamard32_quantize or mx_quantize_transpose).
 * Any pair of formats is accepted.
 * Defined by: FP4-training article on hzrcw.cc, section 02 (the forward,
 * activation-gradient and weight-gradient GEMMs on MX operands); Primus page,
 * sections "性能瓶颈分析" and "GEMM 调优" (GEMM as the dominant training cost).
 * A scale byte 0xFF (E8M0 NaN) makes every output element it contributes to
 * NaN.
 */
mx_status_t mx_gemm(const void *a_codes, const void *a_scales, mx_format_t fa,
                    const void *b_codes, const void *b_scales, mx_format_t fb,
                    int64_t M, int64_t N, int64_t K, void *c, mx_out_t out, int64_t ldc,
                    void *stream);

/*
 * mx_quantize_strided -- mx_quantize with row strides on the outputs: row r's
 * codes go to codes + r * ld_codes and its scales to scales + r * ld_scales
 * (bytes), with ld_codes >= the code bytes of a row (cols, or cols / 2 for
 * E2M1) and ld_scales >= cols / 32.  Codes and scales may share one buffer as
 * long as no byte is written twice: either their extents are disjoint, or
 * ld_codes == ld_scales and each row's scales lie in the gap after its codes.
 *
 * FSDP2 low-precision all-gather payload (MindSpeed-LLM FSDP2 page, section
 * "第 3 步：开启低精度 All-Gather", weights sharded along dim 0 as its
 * "注意事项" requires): a rank quantizes its slab of weight rows [rows x K]
 * (x = its rows, ldx = the full row) into ONE buffer of rows
 *     [ codes (code_bytes(K)) | scales (K / 32) | 0 .. 15 bytes unused ],
 * i.e. codes = payload, scales = payload + code_bytes(K), ld_codes =
 * ld_scales = code_bytes(K) + K / 32 rounded up to a multiple of 16 (no
 * padding when K % 512 == 0; 1.03125 bytes per element for FP8, 0.53125 for
 * E2M1, against 2 for bf16).  K blocks never cross rows, so the
 * ranks' payloads concatenated in rank order -- what an all-gather of one
 * buffer per rank delivers -- are exactly the same layout for the whole
 * weight, bit-identical to quantizing it in one call, and mx_gemm_strided
 * takes them as an operand with those two strides, without a copy.
 * Errors as mx_quantize.
 */
mx_status_t mx_quantize_strided(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx, mx_format_t fmt,
                                void *codes, int64_t ld_codes, void *scales, int64_t ld_scales, void *stream);

/*
 * mx_gemm_strided -- mx_gemm on operands whose rows are strided: row m of A's
 * codes starts at a_codes + m * lda and its scales at a_scales + m * ldsa
 * (bytes), likewise for B with ldb and ldsb; lda >= code bytes of K
 * elements and a multiple of 16 (code rows are read with 16-byte loads; the
 * dense stride always is one), ldsa >= K / 32 (any value).  mx_gemm is the
 * case lda = code bytes of K and ldsa = K / 32.  Used for the gathered FSDP2 payload (see
 * mx_quantize_strided) and for operands that are row slices of larger
 * buffers.  Scale strides that are multiples of 16 bytes, with 16-byte
 * aligned code and dword-aligned scale pointers, keep the pipelined kernel
 * (K % 512 == 0); other strides run the general kernels.
 * Same tolerance as mx_gemm; with the same kernel the results are
 * bit-identical to mx_gemm's on the same values.
 */
mx_status_t mx_gemm_strided(const void *a_codes, int64_t lda, const void *a_scales, int64_t ldsa, mx_format_t fa,
                            const void *b_codes, int64_t ldb, const void *b_scales, int64_t ldsb, mx_format_t fb,
                            int64_t M, int64_t N, int64_t K, void *c, mx_out_t out, int64_t ldc, void *stream);

/*
 * K-panel layout of MX codes -- an alternative storage order of the same
 * codes, chosen by the library for its own transposed quantizers and GEMM
 * (no page prescribes a layout).  The codes of R rows of K elements are K / P
 * panels of R rows x 128 bytes, P = 256 elements for E2M1 and 128 for
 * E4M3 / E5M2: code byte j (j < 128) of row r in panel p is at
 * codes + p * (R * 128) + r * 128 + j, i.e. bytes [128 p, 128 p + 128) of the
 * dense row r.  Same total size as the dense layout; scales stay dense
 * ([R x K/32]).  A transposed quantizer writes each workgroup's codes as
 * whole 32 KiB runs in this order (256 runs of 128 bytes in the dense one),
 * and the GEMM reads both layouts at about the same speed.
 */
typedef enum {
    MX_LAYOUT_ROWS = 0,   /* dense row-major codes, as every other call */
    MX_LAYOUT_PANELS = 1  /* K-panel layout above                        */
} mx_layout_t;

/*
 * mx_quantize_transpose_panels, mx_hadamard32_quantize_panels -- as
 * mx_quantize_transpose and mx_hadamard32_quantize (same codes and scales,
 * same errors), with the codes in the K-panel layout (R = cols output rows,
 * K = rows).  rows must also be a multiple of the panel width: 256 for E2M1,
 * 128 for E4M3 / E5M2 (else MX_ERR_INVALID_ARG).  For callers: the
 * weight-gradient operands that mx_gemm_layout then reads in place.
 */
mx_status_t mx_quantize_transpose_panels(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                                         mx_format_t fmt, void *codes, void *scales, void *stream);
mx_status_t mx_hadamard32_quantize_panels(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                                          uint32_t sign_mask, mx_format_t fmt, void *codes, void *scales,
                                          void *stream);

/*
 * mx_quantize_dual_panels -- mx_quantize_dual (same arguments, codes and
 * scales, same errors) with both forms' codes in the K-panel layout: the
 * row form's (R = rows, K = cols) and the transposed form's (R = cols,
 * K = rows).  cols must be a whole number of fmt_row panels and rows a whole
 * number of fmt_t panels (else MX_ERR_INVALID_ARG).  A workgroup then writes
 * each form as contiguous runs (4 KiB per wave of the row form, 32 KiB of
 * the transposed one).  For callers: a linear layer whose GEMMs all read
 * their operands in place through mx_gemm_layout.
 */
mx_status_t mx_quantize_dual_panels(const void *x_bf16, int64_t rows, int64_t cols, int64_t ldx, mx_format_t fmt_row,
                                    void *codes_row, void *scales_row, mx_format_t fmt_t, int rotate,
                                    uint32_t sign_mask, void *codes_t, void *scales_t, void *stream);

/*
 * mx_gemm_layout -- mx_gemm with each operand's codes in the layout given
 * (a_layout, b_layout); scales dense.  With both MX_LAYOUT_ROWS it is
 * mx_gemm.  A K-panel operand needs the pipelined kernel: K a multiple of
 * 512, 16-byte aligned code and dword-aligned scale pointers, the operand's
 * code bytes below 2^31, and, for an E2M1 operand, an E2M1 partner (beside
 * an FP8 operand an E2M1 stage row is 64 bytes, half a panel row); otherwise
 * MX_ERR_UNSUPPORTED.  Any M and N.  Same computation as mx_gemm: on the
 * same values the results are bit-identical to mx_gemm's with dense
 * operands.  Errors otherwise as mx_gemm (MX_ERR_INVALID_ARG for an unknown
 * layout).
 */
mx_status_t mx_gemm_layout(const void *a_codes, mx_layout_t a_layout, const void *a_scales, mx_format_t fa,
                           const void *b_codes, mx_layout_t b_layout, const void *b_scales, mx_format_t fb,
                           int64_t M, int64_t N, int64_t K, void *c, mx_out_t out, int64_t ldc, void *stream);

/* Static, NUL-terminated name of a status code. */
const char *mx_status_string(mx_status_t s);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int mx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MX_H */
