// gemm.hip -- GEMM over NVFP4 operands on gfx950 matrix cores.
//
// Passes: "Pretraining Large Language Models with NVFP4" (gist.science
// summary), Technische Zusammenfassung 2.B.2 (Fprop, Dgrad, Wgrad GEMMs of a
// linear layer); format 2.A (E2M1 codes, E4M3 scale per 16 elements, FP32
// tensor scale).
//
// The pages' GEMM runs on Blackwell FP4 tensor cores; gfx950's block-scaled
// FP4 MFMA takes power-of-two scales per 32 elements, which cannot express an
// E4M3 scale per 16 elements.  Here every element is decoded to the exact
// fp16 value q * S_b (E2M1 times E4M3 needs at most 6 significant bits and
// lies in [2^-10, 2688], inside fp16's normal range): the hardware converts
// a byte of two codes to an fp16 pair, and one packed fp16 multiply applies
// the block scale.  The fp16 MFMA then accumulates exact products in fp32,
// and the epilogue multiplies by alpha = (1/s_enc_a) (1/s_enc_b).
//
// Both operands are "rows x K" with K contiguous, so one kernel serves all
// passes (the dgrad weight operand is the transposed 16x16-block copy written
// by the quantiser).  A workgroup of 4 waves computes a 256x256 tile; each
// wave owns 128x128 (4x4 MFMA 32x32x16 tiles, 256 fp32 accumulators per lane)
// and decodes its own fragments straight from global memory into registers,
// one 128-wide K step ahead of the MFMAs.  No LDS is used.
//
// Lane layout of v_mfma_f32_32x32x16_f16: lane l supplies row (A) or column
// (B) l % 32 and 8 consecutive k of group l / 32; accumulator j of lane l is
// row (j/4)*8 + (l/32)*4 + j%4, column l % 32.  Within a 128-wide K step the
// lane group g = l / 32 owns k in [64g, 64g + 64): the same permutation of k
// is used for A and B, so the sum is unchanged.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kBM = 256, kBN = 256, kKT = 128;
constexpr int kTM = 4, kTN = 4;  // 32x32 MFMA tiles per wave (128 x 128)

struct Raw {
    uint4 c[4][2];  // per 32-row tile: 32 code bytes (64 k) of this lane's row
    uint32_t s[4];  // per 32-row tile: 4 scale bytes (blocks 4g .. 4g+3 of the step)
};

__device__ __forceinline__ void load_full(const uint8_t* __restrict__ codes,
                                          const uint8_t* __restrict__ scales,
                                          const int64_t (&oc)[4], const int64_t (&os)[4],
                                          int64_t k0, int g, Raw& r)
{
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint4* p = reinterpret_cast<const uint4*>(codes + oc[t] + (k0 >> 1) + 32 * g);
        r.c[t][0] = p[0];
        r.c[t][1] = p[1];
        r.s[t] = *reinterpret_cast<const uint32_t*>(scales + os[t] + (k0 >> 4) + 4 * g);
    }
}

// Last, partial K step: 16-byte granules (two blocks) past the end read as
// zero codes, and scales of blocks past the end read as zero, so their
// products vanish.
__device__ __forceinline__ void load_tail(const uint8_t* __restrict__ codes,
                                          const uint8_t* __restrict__ scales,
                                          const int64_t (&oc)[4], const int64_t (&os)[4],
                                          int64_t k0, int g, int64_t nblk, Raw& r)
{
    const int64_t b0 = (k0 >> 4) + 4 * g;  // first block of this lane's range
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint4* p = reinterpret_cast<const uint4*>(codes + oc[t] + (k0 >> 1) + 32 * g);
        r.c[t][0] = (b0 < nblk) ? p[0] : make_uint4(0, 0, 0, 0);
        r.c[t][1] = (b0 + 2 < nblk) ? p[1] : make_uint4(0, 0, 0, 0);
        uint32_t s = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (b0 + j < nblk) s |= (uint32_t)scales[os[t] + b0 + j] << (8 * j);
        r.s[t] = s;
    }
}

// Eight codes (one dword, k ascending from the low nibble) times the block
// scale pair -> the MFMA fragment, exact in fp16.
__device__ __forceinline__ half8_t decode8(uint32_t w, half2_t ss)
{
    half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    half8_t r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// The four E4M3 scale bytes of a step as fp16 pairs {S_j, S_j}.
__device__ __forceinline__ void scale_pairs(uint32_t s, half2_t (&ss)[4])
{
    half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false);
    half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true);
    ss[0] = __builtin_shufflevector(a, a, 0, 0);
    ss[1] = __builtin_shufflevector(a, a, 1, 1);
    ss[2] = __builtin_shufflevector(b, b, 0, 0);
    ss[3] = __builtin_shufflevector(b, b, 1, 1);
}

__device__ __forceinline__ void compute_step(const Raw& ra, const Raw& rb, float16_t (&acc)[4][4])
{
    half2_t sa[4][4], sb[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        scale_pairs(ra.s[t], sa[t]);
        scale_pairs(rb.s[t], sb[t]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // 8 sub-steps of 16 k (8 per lane group)
        half8_t af[4], bf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4& ca = ra.c[t][i >> 2];
            const uint4& cb = rb.c[t][i >> 2];
            const uint32_t wa = (i & 3) == 0 ? ca.x : (i & 3) == 1 ? ca.y : (i & 3) == 2 ? ca.z : ca.w;
            const uint32_t wb = (i & 3) == 0 ? cb.x : (i & 3) == 1 ? cb.y : (i & 3) == 2 ? cb.z : cb.w;
            af[t] = decode8(wa, sa[t][i >> 1]);
            bf[t] = decode8(wb, sb[t][i >> 1]);
        }
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[tm], bf[tn], acc[tm][tn], 0, 0, 0);
    }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace

template <bool kOutF32>
__global__ __launch_bounds__(256, 1) void k_gemm_nt(
    const uint8_t* __restrict__ a_codes, int64_t a_ldc, const uint8_t* __restrict__ a_scales,
    int64_t a_lds, int a_shift, const float* __restrict__ a_senc,
    const uint8_t* __restrict__ b_codes, int64_t b_ldc, const uint8_t* __restrict__ b_scales,
    int64_t b_lds, int b_shift, const float* __restrict__ b_senc, int64_t M, int64_t N,
    int64_t K, void* __restrict__ c, int64_t ldc)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 5, lr = lane & 31;

    // Tile order: workgroups are dealt round-robin to the 8 XCDs; renumber so
    // that each XCD gets a contiguous range, then walk groups of 8 tile rows
    // column by column so that concurrently running tiles share operand panels.
    const int64_t tiles_m = (M + kBM - 1) / kBM, tiles_n = (N + kBN - 1) / kBN;
    const int64_t T = tiles_m * tiles_n;
    const int64_t hw = blockIdx.x;
    const int64_t L = (T % 8 == 0) ? (hw % 8) * (T / 8) + hw / 8 : hw;
    const int64_t GM = 8;
    const int64_t group = L / (GM * tiles_n);
    const int64_t first_m = group * GM;
    const int64_t gsz = (tiles_m - first_m < GM) ? (tiles_m - first_m) : GM;
    const int64_t in_group = L - group * GM * tiles_n;
    const int64_t tile_m = first_m + in_group % gsz;
    const int64_t tile_n = in_group / gsz;

    const int64_t m0 = tile_m * kBM + (wave >> 1) * 128;
    const int64_t n0 = tile_n * kBN + (wave & 1) * 128;

    int64_t oca[4], osa[4], ocb[4], osb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        int64_t ra = m0 + 32 * t + lr;
        ra = ra < M ? ra : M - 1;
        int64_t rb = n0 + 32 * t + lr;
        rb = rb < N ? rb : N - 1;
        oca[t] = ra * a_ldc;
        osa[t] = (ra >> a_shift) * a_lds;
        ocb[t] = rb * b_ldc;
        osb[t] = (rb >> b_shift) * b_lds;
    }

    float16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int64_t nblk = K >> 4;
    const int64_t nfull = K / kKT;
    Raw ra, rb;
    if (nfull > 0) {
        load_full(a_codes, a_scales, oca, osa, 0, g, ra);
        load_full(b_codes, b_scales, ocb, osb, 0, g, rb);
    }
    for (int64_t s = 0; s < nfull; ++s) {
        Raw na, nb;
        if (s + 1 < nfull) {
            load_full(a_codes, a_scales, oca, osa, (s + 1) * kKT, g, na);
            load_full(b_codes, b_scales, ocb, osb, (s + 1) * kKT, g, nb);
        }
        compute_step(ra, rb, acc);
        ra = na;
        rb = nb;
    }
    if (nfull * kKT < K) {
        load_tail(a_codes, a_scales, oca, osa, nfull * kKT, g, nblk, ra);
        load_tail(b_codes, b_scales, ocb, osb, nfull * kKT, g, nblk, rb);
        compute_step(ra, rb, acc);
    }

    const float alpha = (1.0f / *a_senc) * (1.0f / *b_senc);
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const int64_t col = n0 + 32 * tn + lr;
            if (col >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + 32 * tm + (e >> 2) * 8 + g * 4 + (e & 3);
                if (row >= M) continue;
                const float v = acc[tm][tn][e] * alpha;
                if constexpr (kOutF32)
                    static_cast<float*>(c)[row * ldc + col] = v;
                else
                    static_cast<uint16_t*>(c)[row * ldc + col] = f32_to_bf16_rne(v);
            }
        }
}

// Output of a GEMM with an empty contraction: alpha * 0.
template <bool kOutF32>
__global__ __launch_bounds__(256) void k_fill_zero(void* __restrict__ c, int64_t ldc, int64_t M,
                                                   int64_t N)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= M * N) return;
    const int64_t r = i / N, col = i - r * N;
    if constexpr (kOutF32)
        static_cast<float*>(c)[r * ldc + col] = 0.0f;
    else
        static_cast<uint16_t*>(c)[r * ldc + col] = 0;
}

void launch_gemm_nt(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N, int64_t K,
                    void* c, int64_t ldc, bool out_fp32, hipStream_t s)
{
    if (M == 0 || N == 0) return;
    if (K == 0) {
        dim3 g((unsigned)((M * N + 255) / 256));
        if (out_fp32)
            hipLaunchKernelGGL(k_fill_zero<true>, g, dim3(256), 0, s, c, ldc, M, N);
        else
            hipLaunchKernelGGL(k_fill_zero<false>, g, dim3(256), 0, s, c, ldc, M, N);
        return;
    }
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    dim3 grid((unsigned)tiles), block(256);
    if (out_fp32)
        hipLaunchKernelGGL(k_gemm_nt<true>, grid, block, 0, s, a.codes, a.ld_codes, a.scales,
                           a.ld_scales, a.scale_row_shift, a.s_enc, b.codes, b.ld_codes, b.scales,
                           b.ld_scales, b.scale_row_shift, b.s_enc, M, N, K, c, ldc);
    else
        hipLaunchKernelGGL(k_gemm_nt<false>, grid, block, 0, s, a.codes, a.ld_codes, a.scales,
                           a.ld_scales, a.scale_row_shift, a.s_enc, b.codes, b.ld_codes, b.scales,
                           b.ld_scales, b.scale_row_shift, b.s_enc, M, N, K, c, ldc);
}

}  // namespace nvfp4
