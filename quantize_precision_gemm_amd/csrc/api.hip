// api.hip -- the C ABI declared in include/nvfp4.h: argument validation and
// dispatch to the kernels.  Every check runs on the host before anything is
// enqueued; a failed check returns a negative status and launches nothing.
#include <stdint.h>

#include <mutex>

#include "nvfp4.h"
#include "internal.hpp"

namespace {

using nvfp4::GemmOperand;
using nvfp4::QOut;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// The code layout of a descriptor: a known value, and for the interleaved
// layout code rows of whole 32-byte pieces.
int check_layout(const nvfp4_tensor* t, bool with_t)
{
    if (t->layout == NVFP4_LAYOUT_ROW_MAJOR) return NVFP4_OK;
    if (t->layout != NVFP4_LAYOUT_INTERLEAVED) return NVFP4_ERR_MODE;
    if (t->ld_codes % 32 != 0 || (with_t && t->ld_codes_t % 32 != 0)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

inline bool interleaved(const nvfp4_tensor* t) { return t->layout == NVFP4_LAYOUT_INTERLEAVED; }

int launch_status()
{
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

// Checks of an output descriptor for a rows x cols NVFP4 tensor.
int check_out(const nvfp4_tensor* o, int64_t rows, int64_t cols, int block)
{
    const bool empty = rows == 0 || cols == 0;  // empty tensors need no code buffers
    if (!o || !o->amax || !o->s_enc) return NVFP4_ERR_NULL;
    if (!empty && (!o->codes || !o->scales)) return NVFP4_ERR_NULL;
    if (!aligned(o->codes, 16) || o->ld_codes % 16 != 0) return NVFP4_ERR_ALIGN;
    if (!aligned(o->scales, 4) || o->ld_scales % 4 != 0) return NVFP4_ERR_ALIGN;
    if (!aligned(o->amax, 4) || !aligned(o->s_enc, 4)) return NVFP4_ERR_ALIGN;
    if (o->ld_codes < round_up(cols, 32) / 2 || o->ld_scales < cols / 16) return NVFP4_ERR_SHAPE;
    const int lst = check_layout(o, o->codes_t != nullptr);
    if (lst != NVFP4_OK) return lst;
    if (o->codes_t || o->scales_t) {
        if (block != NVFP4_BLOCK_16X16) return NVFP4_ERR_MODE;
        if (!empty && (!o->codes_t || !o->scales_t)) return NVFP4_ERR_NULL;
        if (!aligned(o->codes_t, 16) || o->ld_codes_t % 16 != 0) return NVFP4_ERR_ALIGN;
        if (!aligned(o->scales_t, 4) || o->ld_scales_t % 4 != 0) return NVFP4_ERR_ALIGN;
        if (o->ld_codes_t < round_up(rows, 32) / 2 || o->ld_scales_t < rows / 16)
            return NVFP4_ERR_SHAPE;
    }
    return NVFP4_OK;
}

QOut qout_of(const nvfp4_tensor* o)
{
    QOut q;
    q.codes = o->codes;
    q.ld_codes = o->ld_codes;
    q.scales = o->scales;
    q.ld_scales = o->ld_scales;
    q.codes_t = o->codes_t;
    q.ld_codes_t = o->ld_codes_t;
    q.scales_t = o->scales_t;
    q.ld_scales_t = o->ld_scales_t;
    q.amax = o->amax;
    q.s_enc = o->s_enc;
    q.il = interleaved(o);
    return q;
}

// A GEMM operand is a descriptor filled by a quantiser: codes, scales and
// s_enc present, shapes consistent with its block layout.
int check_operand(const nvfp4_tensor* t)
{
    if (!t || !t->s_enc) return NVFP4_ERR_NULL;
    if (t->rows > 0 && t->cols > 0 && (!t->codes || !t->scales)) return NVFP4_ERR_NULL;
    if (t->block != NVFP4_BLOCK_1X16 && t->block != NVFP4_BLOCK_16X16) return NVFP4_ERR_MODE;
    if (t->rows < 0 || t->cols < 0 || t->cols % 16 != 0) return NVFP4_ERR_SHAPE;
    if (t->block == NVFP4_BLOCK_16X16 && t->rows % 16 != 0) return NVFP4_ERR_SHAPE;
    if (!aligned(t->codes, 16) || t->ld_codes % 16 != 0) return NVFP4_ERR_ALIGN;
    if (!aligned(t->scales, 4) || t->ld_scales % 4 != 0) return NVFP4_ERR_ALIGN;
    if (t->ld_codes < round_up(t->cols, 32) / 2 || t->ld_scales < t->cols / 16)
        return NVFP4_ERR_SHAPE;
    return check_layout(t, false);
}


// Checks of an MXFP4 descriptor (rows x cols, blocks of 32 along cols).
// need_data: the codes and scales must be present (a non-empty tensor).
int check_mx(const nvfp4_tensor* t, int64_t rows, int64_t cols)
{
    if (!t) return NVFP4_ERR_NULL;
    if (rows > 0 && cols > 0 && (!t->codes || !t->scales)) return NVFP4_ERR_NULL;
    if (t->codes_t || t->scales_t) return NVFP4_ERR_MODE;
    if (t->layout != NVFP4_LAYOUT_ROW_MAJOR) return NVFP4_ERR_MODE;
    if (!aligned(t->codes, 16) || t->ld_codes % 16 != 0) return NVFP4_ERR_ALIGN;
    if (!aligned(t->scales, 4) || t->ld_scales % 4 != 0) return NVFP4_ERR_ALIGN;
    if (t->ld_codes < round_up(cols, 32) / 2 || t->ld_scales < cols / 32) return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t block,
                   int32_t rounding, uint64_t seed, const float* amax_in, nvfp4_tensor* out,
                   void* stream)
{
    if (block != NVFP4_BLOCK_1X16 && block != NVFP4_BLOCK_16X16) return NVFP4_ERR_MODE;
    if (rounding != NVFP4_RNE && rounding != NVFP4_SR) return NVFP4_ERR_MODE;
    if (rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
    if (block == NVFP4_BLOCK_16X16 && rows % 16 != 0) return NVFP4_ERR_SHAPE;
    if (!x && rows > 0 && cols > 0) return NVFP4_ERR_NULL;
    if (ld_x < cols) return NVFP4_ERR_SHAPE;
    if (!aligned(x, 16) || ld_x % 8 != 0) return NVFP4_ERR_ALIGN;
    if (amax_in && !aligned(amax_in, 4)) return NVFP4_ERR_ALIGN;
    int st = check_out(out, rows, cols, block);
    if (st != NVFP4_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const float* amax_src = amax_in;
    if (!amax_src) {
        nvfp4::launch_amax_rows(xb, rows, cols, ld_x, out->amax, s);
        amax_src = out->amax;
    }
    nvfp4::launch_quant(xb, rows, cols, ld_x, block, rounding, seed, amax_src, qout_of(out), s);
    out->rows = rows;
    out->cols = cols;
    out->block = block;
    return launch_status();
}

int nvfp4_rht_quantize(const void* x, int64_t tokens, int64_t channels, int64_t ld_x,
                       uint32_t sign_mask, int32_t rounding, uint64_t seed,
                       const float* amax_in, nvfp4_tensor* out, void* stream)
{
    if (rounding != NVFP4_RNE && rounding != NVFP4_SR) return NVFP4_ERR_MODE;
    if (tokens < 0 || channels < 0 || tokens % 16 != 0 || channels % 8 != 0)
        return NVFP4_ERR_SHAPE;
    if (!x && tokens > 0 && channels > 0) return NVFP4_ERR_NULL;
    if (ld_x < channels) return NVFP4_ERR_SHAPE;
    if (!aligned(x, 16) || ld_x % 8 != 0) return NVFP4_ERR_ALIGN;
    if (amax_in && !aligned(amax_in, 4)) return NVFP4_ERR_ALIGN;
    if (out && (out->codes_t || out->scales_t)) return NVFP4_ERR_MODE;
    int st = check_out(out, channels, tokens, NVFP4_BLOCK_1X16);
    if (st != NVFP4_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint32_t mask = sign_mask & 0xFFFFu;
    const float* amax_src = amax_in;
    if (!amax_src) {
        nvfp4::launch_rht_amax(xb, tokens, channels, ld_x, mask, out->amax, s);
        amax_src = out->amax;
    }
    nvfp4::launch_rht_quant(xb, tokens, channels, ld_x, mask, rounding, seed, amax_src,
                            qout_of(out), s);
    out->rows = channels;
    out->cols = tokens;
    out->block = NVFP4_BLOCK_1X16;
    return launch_status();
}

int nvfp4_quantize_dual(const void* x, int64_t tokens, int64_t channels, int64_t ld_x,
                        uint32_t sign_mask, int32_t rounding, uint64_t seed, uint64_t seed_rht,
                        const float* amax_in, const float* amax_rht_in, nvfp4_tensor* out,
                        nvfp4_tensor* out_rht, void* stream)
{
    if (rounding != NVFP4_RNE && rounding != NVFP4_SR) return NVFP4_ERR_MODE;
    if ((amax_in == nullptr) != (amax_rht_in == nullptr)) return NVFP4_ERR_NULL;
    if (tokens < 0 || channels < 0 || tokens % 16 != 0 || channels % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (!x && tokens > 0 && channels > 0) return NVFP4_ERR_NULL;
    if (ld_x < channels) return NVFP4_ERR_SHAPE;
    if (!aligned(x, 16) || ld_x % 8 != 0) return NVFP4_ERR_ALIGN;
    if (!aligned(amax_in, 4) || !aligned(amax_rht_in, 4)) return NVFP4_ERR_ALIGN;
    if (!out || !out_rht) return NVFP4_ERR_NULL;
    if (out == out_rht) return NVFP4_ERR_MODE;
    if (out->codes_t || out->scales_t || out_rht->codes_t || out_rht->scales_t)
        return NVFP4_ERR_MODE;
    int st = check_out(out, tokens, channels, NVFP4_BLOCK_1X16);
    if (st != NVFP4_OK) return st;
    st = check_out(out_rht, channels, tokens, NVFP4_BLOCK_1X16);
    if (st != NVFP4_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint32_t mask = sign_mask & 0xFFFFu;
    const float* amax_src = amax_in;
    const float* amax_rht_src = amax_rht_in;
    if (!amax_src) {
        nvfp4::launch_amax_dual(xb, tokens, channels, ld_x, mask, out->amax, out_rht->amax, s);
        amax_src = out->amax;
        amax_rht_src = out_rht->amax;
    }
    nvfp4::launch_dual_quant(xb, tokens, channels, ld_x, mask, rounding, seed, seed_rht, amax_src,
                             amax_rht_src, qout_of(out), qout_of(out_rht), s);
    out->rows = tokens;
    out->cols = channels;
    out->block = NVFP4_BLOCK_1X16;
    out_rht->rows = channels;
    out_rht->cols = tokens;
    out_rht->block = NVFP4_BLOCK_1X16;
    return launch_status();
}

int nvfp4_quantize_rht_rows(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t block,
                            uint32_t sign_mask, int32_t rounding, uint64_t seed,
                            const float* amax_in, nvfp4_tensor* out, void* stream)
{
    if (block != NVFP4_BLOCK_1X16 && block != NVFP4_BLOCK_16X16) return NVFP4_ERR_MODE;
    if (rounding != NVFP4_RNE && rounding != NVFP4_SR) return NVFP4_ERR_MODE;
    if (rows < 0 || cols < 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
    if (block == NVFP4_BLOCK_16X16 && rows % 16 != 0) return NVFP4_ERR_SHAPE;
    if (!x && rows > 0 && cols > 0) return NVFP4_ERR_NULL;
    if (ld_x < cols) return NVFP4_ERR_SHAPE;
    if (!aligned(x, 16) || ld_x % 8 != 0) return NVFP4_ERR_ALIGN;
    if (amax_in && !aligned(amax_in, 4)) return NVFP4_ERR_ALIGN;
    int st = check_out(out, rows, cols, block);
    if (st != NVFP4_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint32_t mask = sign_mask & 0xFFFFu;
    const float* amax_src = amax_in;
    if (!amax_src) {
        nvfp4::launch_amax_rows_rht(xb, rows, cols, ld_x, mask, out->amax, s);
        amax_src = out->amax;
    }
    nvfp4::launch_quant_rht_rows(xb, rows, cols, ld_x, block, mask, rounding, seed, amax_src,
                                 qout_of(out), s);
    out->rows = rows;
    out->cols = cols;
    out->block = block;
    return launch_status();
}

int nvfp4_rht_quantize_sized(const void* x, int64_t tokens, int64_t channels, int64_t ld_x,
                             int32_t size, uint64_t signs, int32_t rounding, uint64_t seed,
                             const float* amax_in, nvfp4_tensor* out, void* stream)
{
    if (size != 1 && size != 4 && size != 16 && size != 64) return NVFP4_ERR_MODE;
    if (rounding != NVFP4_RNE && rounding != NVFP4_SR) return NVFP4_ERR_MODE;
    if (tokens < 0 || channels < 0 || tokens % 16 != 0 || tokens % size != 0 || channels % 8 != 0)
        return NVFP4_ERR_SHAPE;
    if (!x && tokens > 0 && channels > 0) return NVFP4_ERR_NULL;
    if (ld_x < channels) return NVFP4_ERR_SHAPE;
    if (!aligned(x, 16) || ld_x % 8 != 0) return NVFP4_ERR_ALIGN;
    if (amax_in && !aligned(amax_in, 4)) return NVFP4_ERR_ALIGN;
    if (out && (out->codes_t || out->scales_t)) return NVFP4_ERR_MODE;
    int st = check_out(out, channels, tokens, NVFP4_BLOCK_1X16);
    if (st != NVFP4_OK) return st;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const float* amax_src = amax_in;
    if (!amax_src) {
        nvfp4::launch_rhtd_amax(xb, tokens, channels, ld_x, size, signs, out->amax, s);
        amax_src = out->amax;
    }
    nvfp4::launch_rhtd_quant(xb, tokens, channels, ld_x, size, signs, rounding, seed, amax_src,
                             qout_of(out), s);
    out->rows = channels;
    out->cols = tokens;
    out->block = NVFP4_BLOCK_1X16;
    return launch_status();
}

int nvfp4_amax(const void* x, int64_t rows, int64_t cols, int64_t ld_x, uint32_t sign_mask,
               float* amax, float* amax_rht, void* stream)
{
    if (rows < 0 || cols < 0 || cols % 8 != 0) return NVFP4_ERR_SHAPE;
    if (amax_rht && rows % 16 != 0) return NVFP4_ERR_SHAPE;
    if (!amax) return NVFP4_ERR_NULL;
    if (!x && rows > 0 && cols > 0) return NVFP4_ERR_NULL;
    if (ld_x < cols) return NVFP4_ERR_SHAPE;
    if (!aligned(x, 16) || ld_x % 8 != 0) return NVFP4_ERR_ALIGN;
    if (!aligned(amax, 4) || (amax_rht && !aligned(amax_rht, 4))) return NVFP4_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (amax_rht)
        nvfp4::launch_amax_dual(xb, rows, cols, ld_x, sign_mask & 0xFFFFu, amax, amax_rht, s);
    else
        nvfp4::launch_amax_rows(xb, rows, cols, ld_x, amax, s);
    return launch_status();
}

// Philox4x32-10 block function on the host (Salmon et al., SC'11).
static void philox_host(uint32_t c[4], uint32_t k0, uint32_t k1)
{
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        c[1] = (uint32_t)p1;
        c[3] = (uint32_t)p0;
        c[0] = n0;
        c[2] = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

uint32_t nvfp4_rht_sign_mask(uint64_t seed)
{
    uint32_t c[4] = {0u, 0u, 0u, 1u};
    philox_host(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    return c[0] & 0xFFFFu;
}

uint64_t nvfp4_rht_signs64(uint64_t seed)
{
    uint32_t c[4] = {0u, 0u, 0u, 1u};
    philox_host(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    return (uint64_t)c[0] | ((uint64_t)c[1] << 32);
}

}  // extern "C"

namespace {

// Validation and operand set-up shared by the two NVFP4 GEMM datapaths.
// Validates the operands of one NVFP4 GEMM pass and resolves them to the
// kernel's A (M x K) and B (N x K) operands.
int resolve_gemm(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, GemmOperand& A,
                 GemmOperand& B, int64_t& M, int64_t& N, int64_t& K)
{
    if (pass != NVFP4_FPROP && pass != NVFP4_DGRAD && pass != NVFP4_WGRAD) return NVFP4_ERR_MODE;
    int st = check_operand(a);
    if (st != NVFP4_OK) return st;
    st = check_operand(b);
    if (st != NVFP4_OK) return st;
    if (a->block != NVFP4_BLOCK_1X16) return NVFP4_ERR_MISMATCH;

    A = GemmOperand{a->codes, a->ld_codes, a->scales, a->ld_scales, 0, a->s_enc, interleaved(a)};
    M = a->rows;
    K = a->cols;
    if (pass == NVFP4_DGRAD) {
        // c = dY (M x N) * W (N x K): W^T (K x N) is the 16x16-block operand
        if (b->block != NVFP4_BLOCK_16X16) return NVFP4_ERR_MISMATCH;
        if (b->rows > 0 && b->cols > 0 && (!b->codes_t || !b->scales_t)) return NVFP4_ERR_NULL;
        if (b->rows != a->cols) return NVFP4_ERR_MISMATCH;
        if (!aligned(b->codes_t, 16) || b->ld_codes_t % 16 != 0) return NVFP4_ERR_ALIGN;
        if (!aligned(b->scales_t, 4) || b->ld_scales_t % 4 != 0) return NVFP4_ERR_ALIGN;
        if (interleaved(b) && b->ld_codes_t % 32 != 0) return NVFP4_ERR_ALIGN;
        if (b->ld_codes_t < round_up(b->rows, 32) / 2 || b->ld_scales_t < b->rows / 16)
            return NVFP4_ERR_SHAPE;
        B = GemmOperand{b->codes_t, b->ld_codes_t, b->scales_t, b->ld_scales_t, 4, b->s_enc,
                        interleaved(b)};
        N = b->cols;
    } else {
        if (b->cols != a->cols) return NVFP4_ERR_MISMATCH;
        if (pass == NVFP4_WGRAD && b->block != NVFP4_BLOCK_1X16) return NVFP4_ERR_MISMATCH;
        B = GemmOperand{b->codes, b->ld_codes, b->scales, b->ld_scales,
                        b->block == NVFP4_BLOCK_16X16 ? 4 : 0, b->s_enc, interleaved(b)};
        N = b->rows;
    }
    // the kernels address an operand's codes and scales with 32-bit offsets
    const int64_t span = int64_t(1) << 32;
    const int64_t b_scale_rows = B.scale_row_shift ? (N + 15) >> 4 : N;
    const int64_t a_code_rows = A.il ? round_up(M, 4) : M, b_code_rows = B.il ? round_up(N, 4) : N;
    if (a_code_rows * A.ld_codes > span || b_code_rows * B.ld_codes > span || M * A.ld_scales > span ||
        b_scale_rows * B.ld_scales > span)
        return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}

int gemm_nvfp4(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c, int64_t ldc,
               int32_t c_dtype, void* stream, bool fp8_blocks)
{
    if (c_dtype != NVFP4_OUT_BF16 && c_dtype != NVFP4_OUT_FP32) return NVFP4_ERR_MODE;
    GemmOperand A, B;
    int64_t M, N, K;
    const int st = resolve_gemm(pass, a, b, A, B, M, N, K);
    if (st != NVFP4_OK) return st;
    if (!c && M > 0 && N > 0) return NVFP4_ERR_NULL;
    if (!aligned(c, c_dtype == NVFP4_OUT_FP32 ? 16 : 8) || ldc % 4 != 0) return NVFP4_ERR_ALIGN;
    if (ldc < N) return NVFP4_ERR_SHAPE;
    const bool f32 = c_dtype == NVFP4_OUT_FP32;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (fp8_blocks && K > 0)
        nvfp4::launch_gemm_fp8blk(A, B, M, N, K, c, ldc, f32, s);
    else  // (an empty contraction is the same zero fill for both)
        nvfp4::launch_gemm_nt(A, B, M, N, K, c, ldc, f32, s);
    return launch_status();
}

// Compute units of the current device (the tail split sizes its parts to them).
int device_cus()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

// The tail-split GEMM on a workspace of ws_bytes (or, with ws_bytes < 0, just
// the size it needs in *need).
int gemm_split(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c, int64_t ldc,
               int32_t c_dtype, void* ws, int64_t ws_bytes, int64_t* need, void* stream)
{
    GemmOperand A, B;
    int64_t M, N, K;
    int st = resolve_gemm(pass, a, b, A, B, M, N, K);
    if (st != NVFP4_OK) return st;
    int64_t full = 0;
    int split = 1;
    const int64_t bytes = (M > 0 && N > 0 && K > 0) ? nvfp4::splitk_plan(M, N, K, device_cus(), full, split) : 0;
    if (need) *need = bytes;
    if (ws_bytes < 0) return NVFP4_OK;
    if (c_dtype != NVFP4_OUT_BF16 && c_dtype != NVFP4_OUT_FP32) return NVFP4_ERR_MODE;
    if (!c && M > 0 && N > 0) return NVFP4_ERR_NULL;
    if (!aligned(c, c_dtype == NVFP4_OUT_FP32 ? 16 : 8) || ldc % 4 != 0) return NVFP4_ERR_ALIGN;
    if (ldc < N) return NVFP4_ERR_SHAPE;
    if (bytes > 0 && (!ws || ws_bytes < bytes)) return NVFP4_ERR_WORKSPACE;
    if (bytes > 0 && !aligned(ws, 16)) return NVFP4_ERR_ALIGN;
    const bool f32 = c_dtype == NVFP4_OUT_FP32;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (bytes > 0)
        nvfp4::launch_gemm_nt_split(A, B, M, N, K, c, ldc, f32, static_cast<float*>(ws), full, split, s);
    else
        nvfp4::launch_gemm_nt(A, B, M, N, K, c, ldc, f32, s);
    return launch_status();
}

}  // namespace

extern "C" {

int nvfp4_gemm(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
               int64_t ldc, int32_t c_dtype, void* stream)
{
    return gemm_nvfp4(pass, a, b, c, ldc, c_dtype, stream, false);
}

int nvfp4_gemm_split_workspace(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b,
                               int64_t* bytes)
{
    if (!bytes) return NVFP4_ERR_NULL;
    return gemm_split(pass, a, b, nullptr, 0, NVFP4_OUT_BF16, nullptr, -1, bytes, nullptr);
}

int nvfp4_gemm_split(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                     int64_t ldc, int32_t c_dtype, void* workspace, int64_t workspace_bytes,
                     void* stream)
{
    if (workspace_bytes < 0) return NVFP4_ERR_SHAPE;
    return gemm_split(pass, a, b, c, ldc, c_dtype, workspace, workspace_bytes, nullptr, stream);
}

}  // extern "C"

namespace {

// Scratch of nvfp4_gemm_split_noalloc: the split parts' fp32 partial tiles,
// at most 256 KB per compute unit of a 256-CU device.  Each GPU the library
// runs on holds its own copy from the load of the library to the end of the
// process.  On the host `scratch` only names the array: kernels get its
// device address, looked up once per device.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

// The current device's address of `scratch`, looked up with that device
// current on its first use; null on failure.
void* scratch_ptr()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int nvfp4_gemm_split_noalloc(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                             int64_t ldc, int32_t c_dtype, void* stream)
{
    int64_t need = 0;
    int st = gemm_split(pass, a, b, nullptr, 0, NVFP4_OUT_BF16, nullptr, -1, &need, nullptr);
    if (st != NVFP4_OK) return st;
    if (need > kScratchBytes) return NVFP4_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_ptr();
        if (!ws) return NVFP4_ERR_LAUNCH;
    }
    return gemm_split(pass, a, b, c, ldc, c_dtype, ws, need > 0 ? kScratchBytes : 0, nullptr, stream);
}

int nvfp4_gemm_fp8blk(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                      int64_t ldc, int32_t c_dtype, void* stream)
{
    return gemm_nvfp4(pass, a, b, c, ldc, c_dtype, stream, true);
}

int nvfp4_gemm_amax(int32_t pass, const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                    int64_t ldc, uint32_t sign_mask, float* amax_out, float* amax_rht_out,
                    void* stream)
{
    if (pass != NVFP4_FPROP && pass != NVFP4_DGRAD) return NVFP4_ERR_MODE;
    GemmOperand A, B;
    int64_t M, N, K;
    const int st = resolve_gemm(pass, a, b, A, B, M, N, K);
    if (st != NVFP4_OK) return st;
    if (!amax_out || (!c && M > 0 && N > 0)) return NVFP4_ERR_NULL;
    if (!aligned(c, 8) || ldc % 4 != 0 || !aligned(amax_out, 4) || !aligned(amax_rht_out, 4))
        return NVFP4_ERR_ALIGN;
    if (ldc < N) return NVFP4_ERR_SHAPE;
    if (amax_rht_out && M % 16 != 0) return NVFP4_ERR_SHAPE;  // whole 16-token chunks
    nvfp4::launch_gemm_nt_amax(A, B, M, N, K, static_cast<uint16_t*>(c), ldc, amax_out,
                               amax_rht_out, sign_mask & 0xFFFFu, static_cast<hipStream_t>(stream));
    return launch_status();
}

int nvfp4_mx_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x, int32_t mode,
                      uint32_t sign_mask, int32_t rounding, uint64_t seed, nvfp4_tensor* out,
                      void* stream)
{
    if (mode != NVFP4_MX_ROWS && mode != NVFP4_MX_COLS && mode != NVFP4_MX_COLS_RHT)
        return NVFP4_ERR_MODE;
    if (rounding != NVFP4_RNE && rounding != NVFP4_SR) return NVFP4_ERR_MODE;
    if (rows < 0 || cols < 0) return NVFP4_ERR_SHAPE;
    if (mode == NVFP4_MX_ROWS && cols % 32 != 0) return NVFP4_ERR_SHAPE;
    if (mode != NVFP4_MX_ROWS && (rows % 32 != 0 || cols % 8 != 0)) return NVFP4_ERR_SHAPE;
    if (!x && rows > 0 && cols > 0) return NVFP4_ERR_NULL;
    if (ld_x < cols) return NVFP4_ERR_SHAPE;
    if (!aligned(x, 16) || ld_x % 8 != 0) return NVFP4_ERR_ALIGN;
    const int64_t orows = mode == NVFP4_MX_ROWS ? rows : cols;
    const int64_t ocols = mode == NVFP4_MX_ROWS ? cols : rows;
    int st = check_mx(out, orows, ocols);
    if (st != NVFP4_OK) return st;

    QOut q{};
    q.codes = out->codes;
    q.ld_codes = out->ld_codes;
    q.scales = out->scales;
    q.ld_scales = out->ld_scales;
    nvfp4::launch_mx_quant(static_cast<const uint16_t*>(x), rows, cols, ld_x, mode,
                           sign_mask & 0xFFFFu, rounding, seed, q, static_cast<hipStream_t>(stream));
    out->rows = orows;
    out->cols = ocols;
    out->block = NVFP4_BLOCK_MX32;
    return launch_status();
}

int nvfp4_mx_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c, int64_t ldc,
                  int32_t c_dtype, void* stream)
{
    if (c_dtype != NVFP4_OUT_BF16 && c_dtype != NVFP4_OUT_FP32) return NVFP4_ERR_MODE;
    if (!a || !b) return NVFP4_ERR_NULL;
    if (a->block != NVFP4_BLOCK_MX32 || b->block != NVFP4_BLOCK_MX32) return NVFP4_ERR_MISMATCH;
    if (a->rows < 0 || b->rows < 0 || a->cols < 0 || a->cols % 32 != 0) return NVFP4_ERR_SHAPE;
    if (b->cols != a->cols) return NVFP4_ERR_MISMATCH;
    int st = check_mx(a, a->rows, a->cols);
    if (st != NVFP4_OK) return st;
    st = check_mx(b, b->rows, b->cols);
    if (st != NVFP4_OK) return st;
    const int64_t M = a->rows, N = b->rows, K = a->cols;
    // the kernel addresses each operand with 32-bit offsets from its base
    const int64_t lim = (int64_t)1 << 32;
    if (M * a->ld_codes >= lim || N * b->ld_codes >= lim || M * a->ld_scales >= lim ||
        N * b->ld_scales >= lim)
        return NVFP4_ERR_SHAPE;
    if (!c && M > 0 && N > 0) return NVFP4_ERR_NULL;
    if (!aligned(c, c_dtype == NVFP4_OUT_FP32 ? 16 : 8) || ldc % 4 != 0) return NVFP4_ERR_ALIGN;
    if (ldc < N) return NVFP4_ERR_SHAPE;
    const GemmOperand A{a->codes, a->ld_codes, a->scales, a->ld_scales, 0, nullptr};
    const GemmOperand B{b->codes, b->ld_codes, b->scales, b->ld_scales, 0, nullptr};
    nvfp4::launch_gemm_mx(A, B, M, N, K, c, ldc, c_dtype == NVFP4_OUT_FP32,
                          static_cast<hipStream_t>(stream));
    return launch_status();
}

int nvfp4_bf16_gemm(int32_t pass, const void* a, int64_t lda, const void* b, int64_t ldb,
                    int64_t M, int64_t N, int64_t K, void* c, int64_t ldc, int32_t c_dtype,
                    void* stream)
{
    if (pass != NVFP4_FPROP && pass != NVFP4_DGRAD && pass != NVFP4_WGRAD) return NVFP4_ERR_MODE;
    if (c_dtype != NVFP4_OUT_BF16 && c_dtype != NVFP4_OUT_FP32) return NVFP4_ERR_MODE;
    if (M < 0 || N < 0 || K < 0 || M % 8 || N % 8 || K % 8) return NVFP4_ERR_SHAPE;
    // rows x columns of a, b and c for the pass
    const int64_t a_cols = pass == NVFP4_FPROP ? K : N;
    const int64_t b_cols = K;
    const int64_t a_rows = M, b_rows = pass == NVFP4_WGRAD ? M : N;
    const int64_t c_rows = pass == NVFP4_WGRAD ? N : M;
    const int64_t c_cols = pass == NVFP4_FPROP ? N : K;
    if ((a_rows > 0 && a_cols > 0 && !a) || (b_rows > 0 && b_cols > 0 && !b)) return NVFP4_ERR_NULL;
    if (c_rows > 0 && c_cols > 0 && !c) return NVFP4_ERR_NULL;
    if (!aligned(a, 16) || !aligned(b, 16) || lda % 8 || ldb % 8) return NVFP4_ERR_ALIGN;
    if (!aligned(c, c_dtype == NVFP4_OUT_FP32 ? 16 : 8) || ldc % 4 != 0) return NVFP4_ERR_ALIGN;
    if (lda < a_cols || ldb < b_cols || ldc < c_cols) return NVFP4_ERR_SHAPE;

    const uint16_t* A = static_cast<const uint16_t*>(a);
    const uint16_t* B = static_cast<const uint16_t*>(b);
    const bool f32 = c_dtype == NVFP4_OUT_FP32;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (pass == NVFP4_FPROP)  // rows of X and of W, both K-contiguous
        nvfp4::launch_bf16_gemm(A, lda, false, B, ldb, false, M, N, K, c, ldc, f32, s);
    else if (pass == NVFP4_DGRAD)  // rows of dY (N-contiguous); W read as N x K, k-contiguous
        nvfp4::launch_bf16_gemm(A, lda, false, B, ldb, true, M, K, N, c, ldc, f32, s);
    else  // both operands contracted over tokens, their rows contiguous
        nvfp4::launch_bf16_gemm(A, lda, true, B, ldb, true, N, K, M, c, ldc, f32, s);
    return launch_status();
}

int nvfp4_mfma_sustain(int64_t blocks, int64_t iters, int32_t operands, float* out, void* stream)
{
    if (!out) return NVFP4_ERR_NULL;
    if (blocks < 1 || blocks > (int64_t(1) << 20) || iters < 1 || iters > (int64_t(1) << 20))
        return NVFP4_ERR_SHAPE;
    if (operands < 0 || operands > 2) return NVFP4_ERR_MODE;
    if (!aligned(out, 4)) return NVFP4_ERR_ALIGN;
    nvfp4::launch_mfma_sustain(blocks, iters, operands, out, static_cast<hipStream_t>(stream));
    return launch_status();
}

const char* nvfp4_status_string(int32_t status)
{
    switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "null pointer";
    case NVFP4_ERR_SHAPE: return "invalid shape";
    case NVFP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case NVFP4_ERR_MODE: return "unknown mode";
    case NVFP4_ERR_MISMATCH: return "operands inconsistent with the pass";
    case NVFP4_ERR_LAUNCH: return "kernel launch failed";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
    }
}

}  // extern "C"
