// gemm_fp8blk.hip -- the second GEMM datapath for NVFP4 operands on gfx950:
// FP8 MFMA over one 16-element block at a time, block scales applied to the
// fp32 partial sums in VALU.
//
// Passes and format: "Pretraining Large Language Models with NVFP4"
// (gist.science summary), Technische Zusammenfassung 2.A (E2M1 codes, one
// E4M3 scale per 16 elements, FP32 tensor scale) and 2.B.2 (Fprop, Dgrad,
// Wgrad).
//
// Every E2M1 value is an E4M3 value, so the codes convert to FP8 exactly
// (a byte lookup).  v_mfma_f32_32x32x16_fp8_fp8 contracts exactly one block
// (K = 16) per instruction: P = sum over the block of q_a q_b, exact in fp32
// (products are multiples of 1/4 up to 36, 16 of them).  The block's scales
// then enter per output element: acc += P * (S_a[m] S_b[n]), where
// S_a S_b (two E4M3 values) and P * S_a S_b are exact in fp32, so only the
// accumulation across blocks rounds.  The epilogue multiplies by
// alpha = (1/s_enc_a)(1/s_enc_b).
//
// Cost on gfx950: per MFMA (one 32x32 tile, one block) every lane updates 16
// accumulators with a multiply and a fused multiply-add -- 32 VALU
// instructions per MFMA, several times the MFMA's own issue time -- so this
// datapath is VALU-bound by construction.  It is kept to be measured beside
// the fp16-decode datapath of gemm.hip (nvfp4_gemm).
//
// Structure: a workgroup of 4 waves computes a 128x128 tile (64x64 per wave,
// 2x2 MFMA tiles) in K steps of 64 (4 blocks).  Per step each thread brings
// 16 code bytes of one A row and one B row into LDS as FP8 bytes, and 128
// threads bring one row's 4 block scales of A or B as fp32; two LDS stages
// alternate, with the next step's global loads issued before the current
// step's MFMAs.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kT = 128;        // tile rows (A) and columns (B)
constexpr int kKS = 64;        // K step: 4 blocks
constexpr int kRow = 72;       // LDS bytes per row: 64 FP8 codes + 8 pad
constexpr int kOp = kT * kRow;

// 8 E2M1 codes (one dword, low nibble first) -> 8 E4M3 bytes of the same
// values.  Magnitude byte from a lookup through v_perm_b32 (codes 0..7 ->
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 in E4M3), sign bit moved from bit 3 to bit 7.
__device__ __forceinline__ uint2 e2m1x8_to_e4m3(uint32_t w)
{
    const uint32_t lut_lo = 0x3C383000u, lut_hi = 0x4C484440u;
    uint2 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t x = (w >> (16 * h)) & 0xFFFFu;           // 4 nibbles
        uint32_t t = ((x & 0xFF00u) << 8) | (x & 0xFFu);    // bytes 0, 2: two nibbles each
        t = ((t & 0x00F000F0u) << 4) | (t & 0x000F000Fu);   // one nibble per byte
        const uint32_t mag = __builtin_amdgcn_perm(lut_hi, lut_lo, t & 0x07070707u);
        const uint32_t v = mag | ((t & 0x08080808u) << 4);
        if (h == 0) r.x = v; else r.y = v;
    }
    return r;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

struct Row16 {   // one thread's share of a step: 16 code bytes of A and of B, 4 scales
    uint4 ca, cb;
    uint32_t s;
};

}  // namespace

template <bool kOutF32>
__global__ __launch_bounds__(256, 2) void k_gemm_fp8blk(GemmOperand A, GemmOperand B, int64_t M,
                                                     int64_t N, int64_t K, void* __restrict__ c,
                                                     int64_t ldc)
{
    __shared__ __attribute__((aligned(16))) uint8_t codes[2][2][kOp];  // [stage][A/B]
    __shared__ __attribute__((aligned(16))) float scl[2][2][4][kT];    // [stage][A/B][block][row]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, lr = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;

    // Tiles in groups of 8 tile rows, walked column by column.
    const int64_t tiles_m = (M + kT - 1) / kT, tiles_n = (N + kT - 1) / kT;
    const int64_t L = blockIdx.x, GM = 8;
    const int64_t group = L / (GM * tiles_n), first_m = group * GM;
    const int64_t gsz = (tiles_m - first_m < GM) ? (tiles_m - first_m) : GM;
    const int64_t in_group = L - group * GM * tiles_n;
    const int64_t tile_m = first_m + in_group % gsz, tile_n = in_group / gsz;

    // thread t: code half t % 2 of tile row t / 2 of A and of B; scales of
    // A row t (t < 128) or B row t - 128
    const int crow = tid >> 1, chalf = tid & 1;
    int64_t ra = tile_m * kT + crow, rb = tile_n * kT + crow;
    ra = ra < M ? ra : M - 1;
    rb = rb < N ? rb : N - 1;
    const uint8_t* pa = A.codes + code_offset(ra, 16 * chalf, A.ld_codes, A.il);
    const uint8_t* pb = B.codes + code_offset(rb, 16 * chalf, B.ld_codes, B.il);
    const int64_t ka = A.il ? 128 : 32, kb = B.il ? 128 : 32;  // code bytes per K step of a row
    const bool s_is_b = tid >= kT;
    int64_t rs = (s_is_b ? tile_n : tile_m) * kT + (tid & (kT - 1));
    rs = rs < (s_is_b ? N : M) ? rs : (s_is_b ? N : M) - 1;
    const GemmOperand& SO = s_is_b ? B : A;
    const uint8_t* ps = SO.scales + (rs >> SO.scale_row_shift) * SO.ld_scales;
    const int64_t nblk = K >> 4;

    auto load = [&](int64_t step, Row16& r) {
        const int64_t b0 = step * 4;
        if (b0 + 4 <= nblk) {
            r.ca = *reinterpret_cast<const uint4*>(pa + ka * step);
            r.cb = *reinterpret_cast<const uint4*>(pb + kb * step);
            r.s = *reinterpret_cast<const uint32_t*>(ps + b0);
        } else {  // partial last step: blocks past K get zero codes and scales
            const bool in = b0 + 2 * chalf < nblk;  // this thread's two blocks
            r.ca = in ? *reinterpret_cast<const uint4*>(pa + ka * step) : make_uint4(0, 0, 0, 0);
            r.cb = in ? *reinterpret_cast<const uint4*>(pb + kb * step) : make_uint4(0, 0, 0, 0);
            r.s = 0u;
            for (int j = 0; j < 4; ++j)
                if (b0 + j < nblk) r.s |= (uint32_t)ps[b0 + j] << (8 * j);
        }
    };
    auto put = [&](const Row16& r, int st) {
        uint8_t* da = &codes[st][0][crow * kRow + 32 * chalf];
        uint8_t* db = &codes[st][1][crow * kRow + 32 * chalf];
        const uint32_t wa[4] = {r.ca.x, r.ca.y, r.ca.z, r.ca.w};
        const uint32_t wb[4] = {r.cb.x, r.cb.y, r.cb.z, r.cb.w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            *reinterpret_cast<uint2*>(da + 8 * d) = e2m1x8_to_e4m3(wa[d]);
            *reinterpret_cast<uint2*>(db + 8 * d) = e2m1x8_to_e4m3(wb[d]);
        }
        const half2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.s, 1.0f, false);
        const half2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.s, 1.0f, true);
        float* sd = &scl[st][s_is_b ? 1 : 0][0][tid & (kT - 1)];
        sd[0 * kT] = (float)s01[0];
        sd[1 * kT] = (float)s01[1];
        sd[2 * kT] = (float)s23[0];
        sd[3 * kT] = (float)s23[1];
    };

    float16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    auto compute = [&](int st) {
#pragma unroll 1
        for (int b = 0; b < 4; ++b) {   // one block at a time bounds the live partials
            long fa[2], fb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                fa[t] = *reinterpret_cast<const long*>(&codes[st][0][(wm * 64 + 32 * t + lr) * kRow + 16 * b + 8 * g]);
                fb[t] = *reinterpret_cast<const long*>(&codes[st][1][(wn * 64 + 32 * t + lr) * kRow + 16 * b + 8 * g]);
            }
            float sb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) sb[t] = scl[st][1][b][wn * 64 + 32 * t + lr];
#pragma unroll
            for (int tm = 0; tm < 2; ++tm) {
                float sa[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = *reinterpret_cast<const float4*>(&scl[st][0][b][wm * 64 + 32 * tm + 8 * q + 4 * g]);
                    sa[4 * q + 0] = v.x;
                    sa[4 * q + 1] = v.y;
                    sa[4 * q + 2] = v.z;
                    sa[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
                    const float16_t zero = {};
                    const float16_t p = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(fa[tm], fb[tn], zero, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[tm][tn][e] = __builtin_fmaf(p[e], sa[e] * sb[tn], acc[tm][tn][e]);
                }
            }
        }
    };

    const int64_t nsteps = (K + kKS - 1) / kKS;
    Row16 r;
    if (nsteps > 0) {
        load(0, r);
        put(r, 0);
    }
    __syncthreads();
    for (int64_t s = 0; s < nsteps; ++s) {
        const int st = (int)(s & 1);
        if (s + 1 < nsteps) load(s + 1, r);
        compute(st);
        if (s + 1 < nsteps) put(r, st ^ 1);
        __syncthreads();
    }

    float alpha;
    int alpha_exp;  // alpha * 2^alpha_exp is the output scale (output_scale)
    output_scale(*A.s_enc, *B.s_enc, alpha, alpha_exp);
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
            const int64_t col = tile_n * kT + wn * 64 + 32 * tn + lr;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = tile_m * kT + wm * 64 + 32 * tm + (e >> 2) * 8 + g * 4 + (e & 3);
                if (row < M && col < N) {
                    float v = acc[tm][tn][e] * alpha;
                    if (alpha_exp != 0) v = __builtin_ldexpf(v, alpha_exp);
                    if constexpr (kOutF32)
                        static_cast<float*>(c)[row * ldc + col] = v;
                    else
                        static_cast<uint16_t*>(c)[row * ldc + col] = f32_to_bf16_rne(v);
                }
            }
        }
}

void launch_gemm_fp8blk(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N,
                        int64_t K, void* c, int64_t ldc, bool out_fp32, hipStream_t s)
{
    if (M == 0 || N == 0 || K == 0) return;  // K == 0 is handled by the caller
    const int64_t tiles = ((M + kT - 1) / kT) * ((N + kT - 1) / kT);
    const dim3 grid((unsigned)tiles), block(256);
    if (out_fp32)
        hipLaunchKernelGGL(k_gemm_fp8blk<true>, grid, block, 0, s, a, b, M, N, K, c, ldc);
    else
        hipLaunchKernelGGL(k_gemm_fp8blk<false>, grid, block, 0, s, a, b, M, N, K, c, ldc);
}

}  // namespace nvfp4
