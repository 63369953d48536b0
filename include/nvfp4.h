/*
 * nvfp4.h -- C ABI of the NVFP4 quantize -> GEMM library for MI355X (gfx950).
 *
 * The library computes the data-parallel hot path of a linear layer trained
 * with the NVFP4 recipe described on the pages about NVIDIA's report
 * "Pretraining Large Language Models with NVFP4" (gist.science summary of that
 * title, "Technische Zusammenfassung" sections 2.A and 2.B):
 *   - NVFP4 tensors: 4-bit E2M1 elements in 16-element blocks, one E4M3 scale
 *     per block and one FP32 scale per tensor (section 2.A);
 *   - weights use 16x16 blocks so that forward and backward see the same
 *     quantised values (section 2.B.3);
 *   - the inputs of the weight-gradient GEMM get a 16-point random Hadamard
 *     transform (section 2.B.2);
 *   - gradients are rounded stochastically, everything else to nearest even
 *     (section 2.B.4);
 *   - GEMMs for the forward (fprop), activation-gradient (dgrad) and
 *     weight-gradient (wgrad) passes (section 2.B.2 names all three).
 *
 * Conventions for every entry point:
 *   - Every data pointer is a DEVICE pointer on the current HIP device and is
 *     owned by the caller, who keeps it alive until the work queued on
 *     `stream` has finished.  `nvfp4_tensor*` arguments are HOST pointers to
 *     descriptors of device buffers.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).  The
 *     calls only enqueue work: they never synchronise, never allocate device
 *     or host memory, and keep no state between calls, so they are reentrant.
 *   - All argument checks happen on the host before anything is enqueued; a
 *     failed check returns a negative status and enqueues nothing.
 *   - Inputs must be finite; NaN or Inf inputs give unspecified codes.
 *   - bf16 data is passed as its 16-bit patterns (uint16).
 *   - Packed codes: element (r, c) of a rows x cols NVFP4 matrix is the
 *     4-bit code in byte j = c / 2 of code row r, low nibble for even c;
 *     where that byte lies is the tensor's code layout (nvfp4_tensor.layout:
 *     codes[r * ld_codes + j] in the row-major layout).
 *     Code = sign << 3 | exponent << 1 | mantissa (OCP E2M1: values 0, 0.5,
 *     1, 1.5, 2, 3, 4, 6).  Scales are OCP E4M3 bytes (bias 7, max 448).
 *   - The value an NVFP4 element stands for is  e2m1(code) * e4m3(scale) /
 *     s_enc.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define NVFP4_OK 0
#define NVFP4_ERR_NULL (-1)     /* a required pointer is NULL */
#define NVFP4_ERR_SHAPE (-2)    /* a size is negative or breaks a multiple-of rule */
#define NVFP4_ERR_ALIGN (-3)    /* a pointer or leading dimension is misaligned */
#define NVFP4_ERR_MODE (-4)     /* unknown block, rounding, pass or dtype */
#define NVFP4_ERR_MISMATCH (-5) /* GEMM operands inconsistent with the pass */
#define NVFP4_ERR_LAUNCH (-6)   /* the HIP runtime reported a launch error */
#define NVFP4_ERR_WORKSPACE (-7) /* the workspace is missing or smaller than needed */

/* Block layouts. */
#define NVFP4_BLOCK_1X16 0      /* one scale per 16 consecutive elements of a row */
#define NVFP4_BLOCK_16X16 1     /* one scale per 16x16 tile (weights) */
#define NVFP4_BLOCK_MX32 2      /* MXFP4: one UE8M0 scale per 32 elements of a row */

/* MXFP4 quantiser layouts (nvfp4_mx_quantize). */
#define NVFP4_MX_ROWS 0         /* blocks along the rows of x; result rows x cols */
#define NVFP4_MX_COLS 1         /* the transposed matrix; result cols x rows */
#define NVFP4_MX_COLS_RHT 2     /* as NVFP4_MX_COLS after the 16-point RHT */

/* Rounding of the elements. */
#define NVFP4_RNE 0             /* round to nearest, ties to even */
#define NVFP4_SR 1              /* stochastic rounding, Philox4x32-10 */

/* GEMM passes. */
#define NVFP4_FPROP 0
#define NVFP4_DGRAD 1
#define NVFP4_WGRAD 2

/* Output element types. */
#define NVFP4_OUT_BF16 0
#define NVFP4_OUT_FP32 1

/* Code layouts (nvfp4_tensor.layout; the scales are row-major in both). */
#define NVFP4_LAYOUT_ROW_MAJOR 0   /* byte j of code row r at r * ld + j */
#define NVFP4_LAYOUT_INTERLEAVED 1 /* rows interleaved by 4 in 32-byte pieces (below) */

/*
 * Descriptor of an NVFP4 tensor (rows x cols, blocks along cols).
 * The caller allocates the buffers and fills the pointer and leading
 * dimension fields; the quantisers fill rows, cols and block.
 *   codes     rows x ld_codes bytes. ld_codes is a multiple of 16 and at
 *             least round_up(cols, 32) / 2; bytes past cols/2 may hold any
 *             value (the GEMM masks them).  16-byte aligned.
 *   scales    1x16 : rows x ld_scales bytes, ld_scales >= cols / 16;
 *             16x16: rows/16 x ld_scales bytes, ld_scales >= cols / 16.
 *             ld_scales is a multiple of 4; 4-byte aligned.
 *   codes_t   optional, 16x16 only: the codes of the transposed matrix
 *             (cols x ld_codes_t bytes, ld_codes_t a multiple of 16 and at
 *             least round_up(rows, 32) / 2).  Needed by the DGRAD GEMM.
 *   scales_t  optional, 16x16 only: the transposed tile scales
 *             (cols/16 x ld_scales_t bytes, ld_scales_t a multiple of 4 and
 *             at least rows / 16).  Needed by the DGRAD GEMM.
 *   amax      1 float: max |x| over the tensor as quantised.
 *   s_enc     1 float: the tensor's FP32 encode scale.
 *   layout    where the bytes of codes and codes_t lie (the caller sets it;
 *             the quantisers write that layout and the GEMMs read it):
 *             NVFP4_LAYOUT_ROW_MAJOR: byte j of code row r at
 *               codes[r * ld_codes + j];
 *             NVFP4_LAYOUT_INTERLEAVED: code rows in groups of 4, each
 *               128-byte piece holding 32 bytes (64 codes) of the 4 rows in
 *               turn: byte j of row r at codes[(r / 4) * 4 * ld_codes +
 *               (j / 32) * 128 + (r % 4) * 32 + j % 32].  ld_codes (and
 *               ld_codes_t) must be a multiple of 32, and codes must hold
 *               round_up(rows, 4) rows (codes_t round_up(cols, 4)); the
 *               padding rows are neither written nor read.  A 64-element K
 *               step of 4 rows is then one 128-byte cache line, which the
 *               NVFP4 GEMMs read whole (the row-major layout makes them touch
 *               a quarter of a line per row and step).
 *             Any other value: NVFP4_ERR_MODE.  The MXFP4 entry points take
 *             the row-major layout only.
 */
typedef struct nvfp4_tensor {
    uint8_t* codes;
    uint8_t* scales;
    uint8_t* codes_t;
    uint8_t* scales_t;
    float* amax;
    float* s_enc;
    int64_t rows;
    int64_t cols;
    int64_t ld_codes;
    int64_t ld_scales;
    int64_t ld_codes_t;
    int64_t ld_scales_t;
    int32_t block;
    int32_t layout;
} nvfp4_tensor;

/*
 * nvfp4_quantize -- NVFP4-quantise a row-major bf16 matrix.
 * Defines: "Pretraining Large Language Models with NVFP4", Technische
 * Zusammenfassung 2.A (format, two-level scaling), 2.B.3 (16x16 blocks for
 * weights), 2.B.4 (RNE for activations and weights, SR for gradients).
 *   x         device bf16, rows x ld_x elements, row-major; 16-byte aligned,
 *             ld_x >= cols and a multiple of 8.
 *   rows      >= 0; a multiple of 16 for NVFP4_BLOCK_16X16.
 *   cols      >= 0 and a multiple of 16 (a block has 16 elements).
 *   block     NVFP4_BLOCK_1X16 or NVFP4_BLOCK_16X16.
 *   rounding  NVFP4_RNE or NVFP4_SR.
 *   seed      Philox key for SR: the 16-bit draw of element (r, c) comes from
 *             counter (r*cols + c) / 8; ignored for RNE.
 *   amax_in   optional device float: if not NULL it is used as the tensor
 *             amax instead of computing one (e.g. a precomputed amax); it is
 *             copied to out->amax.
 *   out       descriptor with codes, scales, amax, s_enc set (and, for
 *             16x16, optionally codes_t / scales_t, which are then written).
 * Tensor scale s_enc = 2688 / amax (1 if amax = 0, FLT_MAX if that
 * overflows); block scale = E4M3(RN(amax_b / 6) * s_enc) rounded to nearest
 * even and saturated at 448; element code = E2M1 rounding of
 * x * (s_enc / scale) (a zero scale gives signed zeros).
 * Returns NVFP4_OK or a negative status.
 */
int nvfp4_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t block,
                   int32_t rounding, uint64_t seed, const float* amax_in, nvfp4_tensor* out,
                   void* stream);

/*
 * nvfp4_rht_quantize -- weight-gradient operand: 16-point random Hadamard
 * transform along the token dimension, transpose, then 1x16 quantisation.
 * Defines: "Pretraining Large Language Models with NVFP4", Technische
 * Zusammenfassung 2.B.2 (16x16 random Hadamard transform on the inputs of the
 * weight-gradient GEMM only) and 2.B.4 (SR for gradients).
 *   x         device bf16, tokens x ld_x elements (row = token); 16-byte
 *             aligned, ld_x >= channels and a multiple of 8.
 *   tokens    >= 0, a multiple of 16 (the transform acts on aligned
 *             16-token chunks).
 *   channels  >= 0, a multiple of 8.
 *   sign_mask bit i set means the i-th sign of the random diagonal is -1.
 *             The transform of a chunk v is (1/4) * H16 * diag(d) * v with
 *             H16 the Sylvester Hadamard matrix, evaluated as a radix-2
 *             butterfly (strides 1, 2, 4, 8) in fp32.  Use the same mask for
 *             both operands of one weight-gradient GEMM.
 *   rounding, seed, amax_in  as for nvfp4_quantize; SR draws are indexed by
 *             c * tokens + t in the transposed layout; amax is taken over the
 *             transformed values.
 *   out       1x16 descriptor of the channels x tokens result.
 */
int nvfp4_rht_quantize(const void* x, int64_t tokens, int64_t channels, int64_t ld_x,
                       uint32_t sign_mask, int32_t rounding, uint64_t seed,
                       const float* amax_in, nvfp4_tensor* out, void* stream);

/*
 * nvfp4_quantize_dual -- both NVFP4 operands of one tensor from a single read:
 * the 1x16 quantisation along the channels (the fprop operand X or the dgrad
 * operand dY) and the RHT-transposed 1x16 quantisation along the tokens (the
 * wgrad operand).
 * Defines: "Pretraining Large Language Models with NVFP4", Technische
 * Zusammenfassung 2.B.2 (the same activation and gradient enter fprop/dgrad
 * untransformed and wgrad after the 16x16 random Hadamard transform) and
 * 2.B.4 (SR for gradients, RNE otherwise; one rounding mode for both results,
 * since both come from the same tensor).
 * The results are bit-identical to
 *   nvfp4_quantize(x, tokens, channels, ld_x, NVFP4_BLOCK_1X16, rounding,
 *                  seed, amax_in, out)
 *   nvfp4_rht_quantize(x, tokens, channels, ld_x, sign_mask, rounding,
 *                      seed_rht, amax_rht_in, out_rht)
 * and cost one read of x instead of two.
 *   x          device bf16, tokens x ld_x elements (row = token); 16-byte
 *              aligned, ld_x >= channels and a multiple of 8.
 *   tokens     >= 0, a multiple of 16.   channels >= 0, a multiple of 16.
 *   sign_mask  as for nvfp4_rht_quantize.
 *   seed       Philox key of the SR draws of out (indexed as in
 *              nvfp4_quantize); seed_rht the key of out_rht's draws.
 *   amax_in, amax_rht_in  both NULL (one nvfp4_amax-style pass computes both
 *              maxima) or both device floats holding max |x| and max |RHT(x)|.
 *   out        1x16 descriptor of the tokens x channels result (no codes_t).
 *   out_rht    1x16 descriptor of the channels x tokens result (no codes_t);
 *              a different descriptor from out, with non-overlapping buffers.
 * Returns NVFP4_OK or a negative status; nothing is launched on error.
 */
int nvfp4_quantize_dual(const void* x, int64_t tokens, int64_t channels, int64_t ld_x,
                        uint32_t sign_mask, int32_t rounding, uint64_t seed, uint64_t seed_rht,
                        const float* amax_in, const float* amax_rht_in, nvfp4_tensor* out,
                        nvfp4_tensor* out_rht, void* stream);

/*
 * nvfp4_quantize_rht_rows -- nvfp4_quantize after the 16-point random
 * Hadamard transform of every aligned 16-element chunk of each row (along
 * the contraction dimension of fprop and dgrad operands).  For the ablation
 * of "Pretraining Large Language Models with NVFP4", Technische
 * Zusammenfassung 2.B.2 (the transform brought no significant benefit on
 * fprop and dgrad, so the recipe keeps it to wgrad).  With one sign mask for
 * both operands of a GEMM the transforms cancel in the product.
 *   Arguments, layout and errors as for nvfp4_quantize; sign_mask as for
 *   nvfp4_rht_quantize; the amax (if not given) is taken over the
 *   transformed values.  With 16x16 blocks an optional transposed copy is
 *   the transpose of the transformed tensor's codes.
 */
int nvfp4_quantize_rht_rows(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t block,
                            uint32_t sign_mask, int32_t rounding, uint64_t seed,
                            const float* amax_in, nvfp4_tensor* out, void* stream);

/*
 * nvfp4_rht_quantize_sized -- nvfp4_rht_quantize with a transform of `size`
 * tokens: 1 (no transform: the plain transposing quantiser), 4, 16 or 64.
 * For the size ablation of "Pretraining Large Language Models with NVFP4",
 * Technische Zusammenfassung 2.B.2 (16 x 16 was the best size for large
 * models).  The D-point transform is the 16-point one generalised: signs,
 * radix-2 butterfly with strides 1 .. D/2 in fp32, then the exact factor
 * 2^-(log2 D / 2); size 16 gives exactly nvfp4_rht_quantize's result.
 *   tokens    a multiple of 16 and of size; channels a multiple of 8.
 *   signs     bit i set: the i-th sign of a chunk is -1 (bits 0 .. size-1
 *             are used; nvfp4_rht_signs64 draws them).
 *   other arguments, layout and errors as for nvfp4_rht_quantize; the amax
 *             (if not given) is taken over the transformed values.
 */
int nvfp4_rht_quantize_sized(const void* x, int64_t tokens, int64_t channels, int64_t ld_x,
                             int32_t size, uint64_t signs, int32_t rounding, uint64_t seed,
                             const float* amax_in, nvfp4_tensor* out, void* stream);

/*
 * nvfp4_rht_signs64 -- host helper: 64 random signs, words 0 (bits 0-31) and
 * 1 (bits 32-63) of the Philox4x32-10 block of nvfp4_rht_sign_mask, whose 16
 * bits are the low 16 here.
 */
uint64_t nvfp4_rht_signs64(uint64_t seed);

/*
 * nvfp4_amax -- tensor amax of a bf16 matrix and, optionally, of its 16-point
 * random Hadamard transform along the rows, in one pass over the data.
 * Defines: "Pretraining Large Language Models with NVFP4", Technische
 * Zusammenfassung 2.A (the FP32 tensor-level scale is taken from the tensor
 * amax) and 2.B.2 (the wgrad inputs are quantised after the transform).
 * A tensor that is quantised twice -- 1x16 for fprop or dgrad and through
 * the RHT for wgrad -- needs both maxima; passing them as amax_in to
 * nvfp4_quantize and nvfp4_rht_quantize replaces their own amax passes with
 * this single read.  The results are identical to those passes' (a maximum
 * does not depend on the order of evaluation).
 *   x         device bf16, rows x ld_x elements, 16-byte aligned, ld_x >= cols
 *             and a multiple of 8; cols a multiple of 8.
 *   amax      device float: max |x|.
 *   amax_rht  device float or NULL: max |RHT(x)| over aligned 16-row chunks
 *             with sign_mask as in nvfp4_rht_quantize (rows = tokens, a
 *             multiple of 16).  NULL skips the transform.
 */
int nvfp4_amax(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint32_t sign_mask,
               float* amax, float* amax_rht, void* stream);

/*
 * nvfp4_rht_sign_mask -- host helper: the 16 random signs of the Hadamard
 * transform drawn from a seed: the low 16 bits of word 0 of
 * Philox4x32-10(key = seed, counter = (0, 0, 0, 1)).
 */
uint32_t nvfp4_rht_sign_mask(uint64_t seed);

/*
 * nvfp4_gemm -- GEMM over NVFP4 operands for the three passes of a linear
 * layer; fp32 accumulation, alpha = 1 / (s_enc(a) * s_enc(b)) applied in the
 * epilogue from the device scalars.
 * Defines: "Pretraining Large Language Models with NVFP4", Technische
 * Zusammenfassung 2.B.2 (Fprop, Dgrad, Wgrad) and 2.B.3 (the weight keeps its
 * quantised values in both passes).
 *   FPROP: a = X  (M x K, 1x16),  b = W (N x K, 1x16 or 16x16)
 *          c[m, n] = sum_k x^[m,k] * w^[n,k]                  (M x N)
 *   DGRAD: a = dY (M x N, 1x16),  b = W (N x K, 16x16 with codes_t, scales_t)
 *          c[m, k] = sum_n dy^[m,n] * w^[n,k]                  (M x K)
 *   WGRAD: a = RHT(dY)^T (N x M), b = RHT(X)^T (K x M), both 1x16 from
 *          nvfp4_rht_quantize with one sign mask
 *          c[n, k] = sum_m a^[n,m] * b^[k,m]                   (N x K)
 *   c         device output, row-major with leading dimension ldc elements;
 *             16-byte aligned (8-byte for BF16), ldc a multiple of 4.
 *   c_dtype   NVFP4_OUT_BF16 (fp32 result rounded to nearest even) or
 *             NVFP4_OUT_FP32.
 * The descriptors must be the ones filled by the quantisers (shapes, block
 * and the device amax/s_enc buffers).  Each operand's codes (rows x
 * ld_codes bytes, for DGRAD's b those of codes_t) and scales span at most
 * 4 GiB (NVFP4_ERR_SHAPE otherwise; the kernels address them with 32-bit
 * offsets).  Returns NVFP4_OK or a negative status.
 */
int nvfp4_gemm(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
               int64_t ldc, int32_t c_dtype, void* stream);

/*
 * nvfp4_gemm_split -- nvfp4_gemm (the same passes, operands, output and
 * validation) with the last wave of output tiles split along the
 * contraction.  Defines: as nvfp4_gemm ("Pretraining Large Language Models
 * with NVFP4", Technische Zusammenfassung 2.B.2, 2.B.3); the split is an
 * order of the fp32 accumulation, which the method leaves free.
 * The output is cut into 256 x 256 tiles, one per workgroup and compute unit.
 * When the tile count is not a multiple of the compute units, the tiles of
 * the last, partial wave are each computed in `split` parts over equal runs
 * of 64-element K steps (split = min(CUs / leftover tiles, 8), each part at
 * least 4 steps), the parts' fp32 sums go to the workspace, and a second
 * kernel adds them in part order, applies alpha and writes c.  The result is
 * deterministic; it may differ from nvfp4_gemm's in the last bits of the
 * fp32 accumulation order (both are within the parity bar of the oracle),
 * and the bf16 output is the round-to-nearest-even of this call's fp32
 * result.  Without a partial wave (or with too short a contraction) it is
 * nvfp4_gemm and touches no workspace.
 *   workspace        device memory, 16-byte aligned, caller-owned, at least
 *                    the size nvfp4_gemm_split_workspace reports for the
 *                    same pass, operands and device; NULL is allowed when
 *                    that size is 0.  Its contents on entry do not matter;
 *                    calls that share a workspace must not overlap.
 *   workspace_bytes  its size; NVFP4_ERR_WORKSPACE if smaller than needed.
 */
int nvfp4_gemm_split(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                     int64_t ldc, int32_t c_dtype, void* workspace, int64_t workspace_bytes,
                     void* stream);

/*
 * nvfp4_gemm_split_workspace -- host query: the workspace bytes
 * nvfp4_gemm_split needs for this pass and these operands on the current
 * device (0 when the tiles fill whole waves).  At most 256 KB per compute
 * unit (64 MiB on 256 CUs).  Validates the operands as nvfp4_gemm does;
 * *bytes is written only on NVFP4_OK.
 */
int nvfp4_gemm_split_workspace(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b,
                               int64_t* bytes);

/*
 * nvfp4_gemm_split_noalloc -- nvfp4_gemm_split without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * split parts go to a 64 MiB array of device memory inside the library
 * (one per GPU, held from the library's load to the end of the process);
 * nothing is allocated by the call.  Same arguments, results and errors as
 * nvfp4_gemm_split; NVFP4_ERR_WORKSPACE if the split needs more than 64 MiB
 * (it needs at most 256 KB per compute unit, 64 MiB on 256 CUs).  The first
 * call on a device looks up that device's address of the array
 * (NVFP4_ERR_LAUNCH if the runtime refuses).  All calls on one GPU share the
 * array: calls that overlap on one GPU (concurrent streams, threads) race
 * and must be serialised by the caller.  The array needs no clearing: every
 * part is written before it is read.
 */
int nvfp4_gemm_split_noalloc(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                             int64_t ldc, int32_t c_dtype, void* stream);

/*
 * nvfp4_gemm_fp8blk -- the same GEMM as nvfp4_gemm (same arguments, passes,
 * validation and result within the same tolerance) by the second datapath:
 * each NVFP4 block of 16 products is contracted by an FP8 matrix-core
 * instruction (E2M1 values are exact in E4M3), and the two block scales
 * multiply the exact fp32 partial before it is accumulated.  Only the
 * accumulation across blocks rounds, in block order.
 * Defines: "Pretraining Large Language Models with NVFP4", Technische
 * Zusammenfassung 2.A (16-element blocks with an E4M3 scale each) and 2.B.2
 * (the three passes).  Slower than nvfp4_gemm on gfx950 (the per-block
 * scaling is vector-ALU work); provided so both datapaths can be measured.
 */
int nvfp4_gemm_fp8blk(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                      int64_t ldc, int32_t c_dtype, void* stream);

/*
 * nvfp4_gemm_amax -- nvfp4_gemm for FPROP or DGRAD with bf16 output whose
 * epilogue also reduces that output to the tensor maxima of its next
 * quantisation: amax_out = max |c| (the amax of the two-level scale) and, if
 * amax_rht_out is given, the amax of c's 16-point random Hadamard transform
 * along its rows (tokens) in aligned 16-row chunks -- the wgrad operand's.
 * Defines: "Pretraining Large Language Models with NVFP4", Technische
 * Zusammenfassung 2.A (the FP32 tensor-level scale comes from the tensor's
 * amax) and 2.B.2 (a layer output becomes the next layer's fprop operand
 * and, after the transform, its wgrad operand).  The codes still need the
 * tensor scale before any block can be encoded, so they come from a second
 * pass: nvfp4_quantize_dual(c, ..., amax_in = amax_out, amax_rht_in =
 * amax_rht_out) then skips its own read for the maxima; both maxima equal
 * nvfp4_amax(c) exactly.
 *   pass, a, b, c, ldc   as for nvfp4_gemm (c is bf16); NVFP4_ERR_MODE for
 *                        WGRAD (its fp32 output is not quantised again).
 *   sign_mask            the transform's signs, as for nvfp4_rht_quantize.
 *   amax_out             device float, required; overwritten.
 *   amax_rht_out         device float or null; overwritten.  With it, the
 *                        output rows must be a multiple of 16
 *                        (NVFP4_ERR_SHAPE).
 * Returns NVFP4_OK or a negative status; nothing is enqueued on failure.
 */
int nvfp4_gemm_amax(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                    int64_t ldc, uint32_t sign_mask, float* amax_out, float* amax_rht_out,
                    void* stream);

/*
 * nvfp4_bf16_gemm -- the three GEMMs of a linear layer that stays in BF16
 * (no quantisation); bf16 products accumulated in fp32.
 * Defines: "Pretraining Large Language Models with NVFP4", Technische
 * Zusammenfassung 2.B.1 (mixed precision: the most sensitive linear layers,
 * the last blocks of the network among them, keep BF16) with the passes of
 * 2.B.2.  M = tokens, K = input features, N = output features; every
 * operand is a row-major bf16 matrix as the layer holds it, and the kernel
 * reads W, X and dY in place (no transposed copies):
 *   FPROP: a = X  (M x K, lda), b = W (N x K, ldb)
 *          c[m, n] = sum_k x[m,k] * w[n,k]                     (M x N)
 *   DGRAD: a = dY (M x N, lda), b = W (N x K, ldb)
 *          c[m, k] = sum_n dy[m,n] * w[n,k]                    (M x K)
 *   WGRAD: a = dY (M x N, lda), b = X (M x K, ldb)
 *          c[n, k] = sum_m dy[m,n] * x[m,k]                    (N x K)
 *   M, N, K   >= 0 and multiples of 8.
 *   a, b      device bf16, 16-byte aligned; lda, ldb (elements) multiples
 *             of 8 and at least the row length of the operand.
 *   c, ldc, c_dtype  as for nvfp4_gemm (the output has no alpha: 1).
 * Returns NVFP4_OK or a negative status; nothing is enqueued on failure.
 */
int nvfp4_bf16_gemm(int32_t pass, const void* a, int64_t lda, const void* b, int64_t ldb,
                    int64_t M, int64_t N, int64_t K, void* c, int64_t ldc, int32_t c_dtype,
                    void* stream);

/*
 * nvfp4_mx_quantize -- MXFP4 quantisation, the format NVFP4 is compared with.
 * Defines: "Pretraining Large Language Models with NVFP4", Technische
 * Zusammenfassung 2.A (MXFP4: E2M1 elements in blocks of 32 sharing one
 * UE8M0 power-of-two scale, no tensor-level scale); the conversion rule is
 * the OCP Microscaling v1.0 one: shared exponent e = floor(log2(amax_b)) - 2
 * clamped to [-127, 127] (-127 for an all-zero block), scale byte e + 127,
 * element code = E2M1 rounding (RNE saturating, or SR as for
 * nvfp4_quantize) of x * 2^-e.
 *   x         device bf16, rows x ld_x elements, row-major; 16-byte aligned,
 *             ld_x >= cols and a multiple of 8.
 *   mode      NVFP4_MX_ROWS: blocks along the rows (cols a multiple of 32);
 *             result rows x cols.
 *             NVFP4_MX_COLS: the transposed matrix, blocks along the columns
 *             of x (rows a multiple of 32, cols of 8); result cols x rows.
 *             NVFP4_MX_COLS_RHT: as NVFP4_MX_COLS after the 16-point random
 *             Hadamard transform of every 16-row chunk of each column, with
 *             sign_mask as in nvfp4_rht_quantize (the wgrad operand, 2.B.2).
 *   rounding, seed  NVFP4_RNE or NVFP4_SR; the draw of result element (r, c)
 *             is indexed r * result_cols + c (2.B.4).
 *   out       descriptor: codes (result rows x ld_codes, as for NVFP4) and
 *             scales (result rows x ld_scales bytes, ld_scales a multiple of
 *             4 and >= result_cols / 32; 4-byte aligned); codes_t and
 *             scales_t must be NULL; amax and s_enc are not used.  rows,
 *             cols and block (NVFP4_BLOCK_MX32) are filled in.
 * Returns NVFP4_OK or a negative status; nothing is launched on error.
 */
int nvfp4_mx_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t mode,
                      uint32_t sign_mask, int32_t rounding, uint64_t seed, nvfp4_tensor* out,
                      void* stream);

/*
 * nvfp4_mx_gemm -- GEMM over MXFP4 operands on gfx950's block-scaled FP4
 * matrix instructions, fp32 accumulation:
 *   c[m, n] = sum_k a^[m, k] * b^[n, k]     (a: M x K, b: N x K, both
 *   MXFP4 with blocks along K; x^ = code value * 2^(scale - 127)).
 * The three passes of a linear layer take operands quantised accordingly:
 * fprop (X, W) with NVFP4_MX_ROWS; dgrad (dY with NVFP4_MX_ROWS, W with
 * NVFP4_MX_COLS); wgrad (dY and X with NVFP4_MX_COLS or NVFP4_MX_COLS_RHT).
 * Defines: the comparison of Technische Zusammenfassung 2.A, measured as the
 * speed of the 2.B.2 GEMMs in the other format.
 *   a, b      MXFP4 descriptors (block NVFP4_BLOCK_MX32) with equal cols = K,
 *             a multiple of 32; each operand's codes (rows x ld_codes) and
 *             scales (rows x ld_scales) span less than 4 GiB.
 *   c, ldc, c_dtype  as for nvfp4_gemm (no alpha: MXFP4 has no tensor scale).
 * Returns NVFP4_OK or a negative status; nothing is enqueued on failure.
 */
int nvfp4_mx_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c, int64_t ldc,
                  int32_t c_dtype, void* stream);

/*
 * nvfp4_mfma_sustain -- measurement aid for the GEMMs' roofline, not a pass
 * of the method: a register-only stream of the matrix instruction a GEMM of
 * this library contracts with (Technische Zusammenfassung 2.B.2 defines the
 * GEMMs, 2.A the MXFP4 comparison; the instructions are this library's
 * choice).  A caller times it to learn the matrix throughput the GPU
 * sustains under load, beside the published peak.
 *   blocks    workgroups of 512 threads (8 waves, two per SIMD), 1 .. 2^20.
 *   iters     rounds per wave, 1 .. 2^20; one round is 64 instructions on a
 *             pool of 8 A and 8 B fragments, a different pair each time.
 *             FLOPs of one call: 2 * 32 * 32 * Kinst * 64 * 8 * iters *
 *             blocks, Kinst = 16 for operands 0 and 1, 64 for operands 2.
 *   operands  0: nvfp4_gemm's v_mfma_f32_32x32x16_f16 on exact fp16 values
 *             e2m1 x e4m3 / 64 with random signs (the kind of value the
 *             GEMM's decode produces); 1: the same instruction on random fp16
 *             in [-1, 1); 2: nvfp4_mx_gemm's block-scaled FP4 instruction
 *             v_mfma_scale_f32_32x32x64_f8f6f4 on random E2M1 codes with
 *             unit scales.
 *   out       device float[blocks * 512], 4-byte aligned: one checksum per
 *             thread (the sum of its accumulators).
 * Returns NVFP4_OK, NVFP4_ERR_NULL (out), NVFP4_ERR_SHAPE (blocks or iters
 * out of range), NVFP4_ERR_MODE (operands) or NVFP4_ERR_ALIGN; nothing is
 * enqueued on failure.
 */
int nvfp4_mfma_sustain(int64_t blocks, int64_t iters, int32_t operands, float* out, void* stream);

/* Human-readable name of a status code (static string). */
const char* nvfp4_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
