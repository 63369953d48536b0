// internal.hpp -- launch functions shared between the C-ABI layer and the
// kernel translation units.  Callers have validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Quantiser outputs (device pointers; codes_t / scales_t may be null).
struct QOut {
    uint8_t* codes;
    int64_t ld_codes;
    uint8_t* scales;
    int64_t ld_scales;
    uint8_t* codes_t;
    int64_t ld_codes_t;
    uint8_t* scales_t;
    int64_t ld_scales_t;
    float* amax;
    float* s_enc;
    bool il;  // codes (and codes_t) 4-row interleaved (code_offset), else row-major
};

// One GEMM operand: rows x K NVFP4 codes with 16-element blocks along K,
// row-major or 4-row interleaved (il; see code_offset).  The scale of block b
// of row r is scales[(r >> scale_row_shift) * ld_scales + b].
struct GemmOperand {
    const uint8_t* codes;
    int64_t ld_codes;
    const uint8_t* scales;
    int64_t ld_scales;
    int scale_row_shift;
    const float* s_enc;
    bool il = false;
};

void launch_amax_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* amax,
                      hipStream_t s);
void launch_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int block,
                  int rounding, uint64_t seed, const float* amax_src, const QOut& o,
                  hipStream_t s);
void launch_rht_amax(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld,
                     uint32_t mask, float* amax, hipStream_t s);
void launch_amax_dual(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld,
                      uint32_t mask, float* amax, float* amax_rht, hipStream_t s);
void launch_rht_quant(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld,
                      uint32_t mask, int rounding, uint64_t seed, const float* amax_src,
                      const QOut& o, hipStream_t s);

// One read of x: o gets the 1x16 quantisation along the channels, o_rht the
// RHT-transposed one (same codes as launch_quant and launch_rht_quant).
void launch_dual_quant(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld,
                       uint32_t mask, int rounding, uint64_t seed, uint64_t seed_rht,
                       const float* amax_src, const float* amax_rht_src, const QOut& o,
                       const QOut& o_rht, hipStream_t s);

// The 16-point RHT on every 16-element row chunk, then the quantisation of
// launch_quant (fprop / dgrad ablation).
void launch_amax_rows_rht(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint32_t mask,
                          float* amax, hipStream_t s);
void launch_quant_rht_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int block,
                           uint32_t mask, int rounding, uint64_t seed, const float* amax_src,
                           const QOut& o, hipStream_t s);

// Sized RHT (size 1, 4, 16 or 64 tokens) + transpose + 1x16 quantisation.
void launch_rhtd_amax(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld, int size,
                      uint64_t signs, float* amax, hipStream_t s);
void launch_rhtd_quant(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld, int size,
                       uint64_t signs, int rounding, uint64_t seed, const float* amax_src,
                       const QOut& o, hipStream_t s);

// MXFP4: mode 0 blocks of 32 along the rows of x; 1 the transposed matrix;
// 2 the transposed matrix after the 16-point RHT (o: codes and scales only).
void launch_mx_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int mode,
                     uint32_t mask, int rounding, uint64_t seed, const QOut& o, hipStream_t s);

// C[m, n] = (1/s_enc_a) (1/s_enc_b) sum_k a^[m, k] b^[n, k]; out_fp32 selects
// fp32 or bf16 (round to nearest even) output.
void launch_gemm_nt(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N,
                    int64_t K, void* c, int64_t ldc, bool out_fp32, hipStream_t s);

// Tail split of launch_gemm_nt: when the tile count leaves the last wave of
// workgroups on `cus` compute units partial, its tiles are split along K so
// that the parts fill that wave.  splitk_plan gives the workspace bytes the
// launch needs (0: no split; then full_tiles is every tile and split 1);
// launch_gemm_nt_split runs the GEMM with that plan and a workspace of at
// least that size (fp32 partial tiles), then adds the parts in order.
int64_t splitk_plan(int64_t M, int64_t N, int64_t K, int cus, int64_t& full_tiles, int& split);
void launch_gemm_nt_split(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N,
                          int64_t K, void* c, int64_t ldc, bool out_fp32, float* ws,
                          int64_t full_tiles, int split, hipStream_t s);

// launch_gemm_nt with bf16 output whose epilogue also writes the output's
// tensor amax (max |c|) and, if amax_rht is not null, the amax of its
// 16-point RHT along the rows (M a multiple of 16); both are zeroed first.
void launch_gemm_nt_amax(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N,
                         int64_t K, uint16_t* c, int64_t ldc, float* amax, float* amax_rht,
                         uint32_t mask, hipStream_t s);

// The same product by the other datapath: FP8 MFMA per 16-element block,
// block scales applied to the fp32 partials (K > 0).
void launch_gemm_fp8blk(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N,
                        int64_t K, void* c, int64_t ldc, bool out_fp32, hipStream_t s);

// C[m, n] = sum_k a^[m, k] b^[n, k] over MXFP4 operands (scales in the
// GemmOperand's scales; s_enc and scale_row_shift unused).
void launch_gemm_mx(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N, int64_t K,
                    void* c, int64_t ldc, bool out_fp32, hipStream_t s);

// C[m, n] = sum_k A[m, k] B[n, k] over bf16 operands; a_t / b_t: the operand
// is stored K x rows (element (r, k) at k * ld + r) instead of rows x K.
// M, N, K are multiples of 8.
void launch_bf16_gemm(const uint16_t* a, int64_t lda, bool a_t, const uint16_t* b, int64_t ldb,
                      bool b_t, int64_t M, int64_t N, int64_t K, void* c, int64_t ldc,
                      bool out_fp32, hipStream_t s);

// Register-only stream of matrix instructions: `blocks` workgroups of 512
// threads, `iters` rounds of 64 instructions per wave; operands 0 = fp16
// 32x32x16 on exact E2M1 x E4M3 fp16 values, 1 = the same on random fp16,
// 2 = block-scaled FP4 32x32x64 on random E2M1 codes; one float per thread
// into out.
void launch_mfma_sustain(int64_t blocks, int64_t iters, int operands, float* out, hipStream_t s);

}  // namespace nvfp4
