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
// by the quantiser).  A workgroup of 8 waves (two per SIMD) computes a
// 256x256 tile in K steps of 64.  Per step each thread decodes one row of A
// (threads 0-255) or of B (256-511) -- 32 code bytes, 4 scales -- into an
// fp16 tile in LDS, so each element is decoded once per workgroup; each wave
// then runs 4x2 MFMA 32x32x16 tiles (a 128x64 slab, 128 fp32 accumulators)
// over the tile.  Two LDS stages alternate: while the MFMAs consume one, the
// next step's codes (loaded from global memory one step earlier) are decoded
// into the other, and the global loads two steps ahead are in flight.  Two
// waves per SIMD let one wave's MFMAs cover the other's waits.  The epilogue
// stages 32 output rows per wave through LDS and stores 16-byte segments.
//
// Lane layout of v_mfma_f32_32x32x16_f16: lane l supplies row (A) or column
// (B) l % 32 and the 8 consecutive k 8*(l/32) .. +7 of the 16-wide step;
// accumulator j of lane l is row (j/4)*8 + (l/32)*4 + j%4, column l % 32.
#include <utility>

#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

constexpr int kBM = 256, kBN = 256, kKS = 64;  // workgroup tile and K step
constexpr int kRowBytes = 144;                 // LDS row: 64 fp16 (128 B) + 16 B pad
constexpr int kOpBytes = 256 * kRowBytes;      // one operand, one stage

// This thread's row of A and of B for one K step: 32 code bytes (64 k) and
// 4 scale bytes each.
struct Stage {
    uint4 ca0, ca1, cb0, cb1;
    uint32_t sa, sb;
};

__device__ __forceinline__ void load_row(const uint8_t* __restrict__ codes,
                                         const uint8_t* __restrict__ scales, int64_t oc,
                                         int64_t os, int64_t k0, int64_t nblk, uint4& c0,
                                         uint4& c1, uint32_t& s)
{
    const int64_t b0 = k0 >> 4;
    const uint4* p = reinterpret_cast<const uint4*>(codes + oc + (k0 >> 1));
    if (b0 + 4 <= nblk) {
        c0 = p[0];
        c1 = p[1];
        s = *reinterpret_cast<const uint32_t*>(scales + os + b0);
    } else {  // partial last step: missing blocks get zero codes and zero scales
        c0 = (b0 < nblk) ? p[0] : make_uint4(0, 0, 0, 0);
        c1 = (b0 + 2 < nblk) ? p[1] : make_uint4(0, 0, 0, 0);
        s = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (b0 + j < nblk) s |= (uint32_t)scales[os + b0 + j] << (8 * j);
    }
}

// Decode 64 codes (4 blocks) of one row to exact fp16 q * S and store them to
// the row's 128 bytes in LDS.
__device__ __forceinline__ void decode_row(const uint4& c0, const uint4& c1, uint32_t s,
                                           uint8_t* __restrict__ dst)
{
    const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, false);
    const half2_t sb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s, 1.0f, true);
    const half2_t ss[4] = {__builtin_shufflevector(sa, sa, 0, 0), __builtin_shufflevector(sa, sa, 1, 1),
                           __builtin_shufflevector(sb, sb, 0, 0), __builtin_shufflevector(sb, sb, 1, 1)};
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int d = 0; d < 8; ++d) {  // dword d: elements 8d .. 8d+7, block d / 2
        const half2_t S = ss[d >> 1];
        half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 1.0f, 0) * S;
        half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 1.0f, 1) * S;
        half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 1.0f, 2) * S;
        half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[d], 1.0f, 3) * S;
        uint4 v;
        v.x = __builtin_bit_cast(uint32_t, p0);
        v.y = __builtin_bit_cast(uint32_t, p1);
        v.z = __builtin_bit_cast(uint32_t, p2);
        v.w = __builtin_bit_cast(uint32_t, p3);
        *reinterpret_cast<uint4*>(dst + 16 * d) = v;
    }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace

// One workgroup (4 waves) computes a 256 x 256 tile.  Per K step of 64:
// every thread decodes one row of A and one row of B into the fp16 LDS
// stage, so each element is decoded once per workgroup; each wave then runs
// 4 x 4 MFMA 32x32x16 tiles (128 x 128) over the stage.  Two LDS stages
// alternate; the global loads of step s+2 are issued before the MFMAs of
// step s, and step s+1 (loaded one iteration earlier) is decoded after them.
// Instruction-schedule hint for one K step (32 MFMAs per wave): the first
// half of the MFMAs is interleaved with the LDS fragment reads only; the
// second half also carries the decode of the next step (4 VALU per MFMA) and
// its LDS writes, which gives the global loads feeding that decode as much
// time as possible to land.
template <int kM>
__device__ __forceinline__ void interleave_slot()
{
    constexpr int sub = kM / 8;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr (kM < 16) {
        if constexpr (sub < 3 && kM % 2 == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    } else {
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
        if constexpr (kM % 2 == 1) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
        if constexpr (sub < 3 && kM % 2 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
}

template <int... kMs>
__device__ __forceinline__ void interleave_step(std::integer_sequence<int, kMs...>)
{
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // fragments of the first sub-step
    (interleave_slot<kMs>(), ...);
}

template <bool kOutF32>
__global__ __launch_bounds__(512, 1) void k_gemm_nt(
    const uint8_t* __restrict__ a_codes, int64_t a_ldc, const uint8_t* __restrict__ a_scales,
    int64_t a_lds, int a_shift, const float* __restrict__ a_senc,
    const uint8_t* __restrict__ b_codes, int64_t b_ldc, const uint8_t* __restrict__ b_scales,
    int64_t b_lds, int b_shift, const float* __restrict__ b_senc, int64_t M, int64_t N,
    int64_t K, void* __restrict__ c, int64_t ldc)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kOpBytes];  // [stage][A/B]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
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

    // the row this thread loads and decodes: threads 0..255 take A rows,
    // 256..511 B rows (clamped; the extra rows are never stored)
    const bool is_b = tid >= 256;
    const int rid = tid & 255;
    int64_t rr = is_b ? tile_n * kBN + rid : tile_m * kBM + rid;
    const int64_t lim = is_b ? N : M;
    rr = rr < lim ? rr : lim - 1;
    const uint8_t* my_codes = is_b ? b_codes : a_codes;
    const uint8_t* my_scales = is_b ? b_scales : a_scales;
    const int64_t oc = rr * (is_b ? b_ldc : a_ldc);
    const int64_t os = (rr >> (is_b ? b_shift : a_shift)) * (is_b ? b_lds : a_lds);

    float16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int64_t nblk = K >> 4;
    const int64_t nsteps = (K + kKS - 1) / kKS;
    const int wm = wave >> 2, wn = wave & 3;
    // fragment read offsets within a stage: row (32 t + lr) of the wave's
    // 128-row A slab / 64-row B slab, k = 16 i + 8 g
    const int a_frag = (wm * 128 + lr) * kRowBytes + 16 * g;
    const int b_frag = (wn * 64 + lr) * kRowBytes + 16 * g;

    auto load = [&](int64_t step, Stage& st) {
        load_row(my_codes, my_scales, oc, os, step * kKS, nblk, st.ca0, st.ca1, st.sa);
    };
    auto decode = [&](const Stage& st, int stage) {
        decode_row(st.ca0, st.ca1, st.sa, &lds[stage][is_b ? 1 : 0][rid * kRowBytes]);
    };
    auto compute = [&](int stage) {
        const uint8_t* As = lds[stage][0];
        const uint8_t* Bs = lds[stage][1];
        half8_t af[2][4], bf[2][2];  // fragments of two sub-steps in flight
#pragma unroll
        for (int t = 0; t < 4; ++t) af[0][t] = *reinterpret_cast<const half8_t*>(As + a_frag + t * 32 * kRowBytes);
#pragma unroll
        for (int t = 0; t < 2; ++t) bf[0][t] = *reinterpret_cast<const half8_t*>(Bs + b_frag + t * 32 * kRowBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cur = i & 1, nxt = cur ^ 1;
            if (i < 3) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    af[nxt][t] = *reinterpret_cast<const half8_t*>(As + a_frag + t * 32 * kRowBytes + 32 * (i + 1));
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    bf[nxt][t] = *reinterpret_cast<const half8_t*>(Bs + b_frag + t * 32 * kRowBytes + 32 * (i + 1));
            }
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cur][tm], bf[cur][tn], acc[tm][tn], 0, 0, 0);
        }
    };

    // Main loop over full K steps (no partial-step code inside it).
    const int64_t nfull = K / kKS;
    auto load_full = [&](int64_t step, Stage& st) {
        const int64_t k0 = step * kKS;
        const uint4* p = reinterpret_cast<const uint4*>(my_codes + oc + (k0 >> 1));
        st.ca0 = p[0];
        st.ca1 = p[1];
        st.sa = *reinterpret_cast<const uint32_t*>(my_scales + os + (k0 >> 4));
    };
    Stage g0, g1;
    if (nfull > 0) {
        load_full(0, g0);
        decode(g0, 0);
        load_full(nfull > 1 ? 1 : 0, g1);
    }
    __syncthreads();
    int64_t s = 0;
    for (; s + 2 <= nfull; s += 2) {
        // even step s: LDS stage 0 holds s, g1 holds s+1, g0 is free
        // unconditional (clamped) loads keep the wait counts exact
        load_full(s + 2 < nfull ? s + 2 : nfull - 1, g0);
        compute(0);
        decode(g1, 1);
        interleave_step(std::make_integer_sequence<int, 32>{});
        __syncthreads();
        // odd step s+1: stage 1 holds s+1, g0 holds s+2, g1 is free
        load_full(s + 3 < nfull ? s + 3 : nfull - 1, g1);
        compute(1);
        decode(g0, 0);  // harmless on the last pass: stage 0 is not read again
        interleave_step(std::make_integer_sequence<int, 32>{});
        __syncthreads();
    }
    if (s < nfull) compute(0);  // odd number of full steps: the last one is in stage 0
    if (nfull < nsteps) {       // partial last step
        load(nfull, g1);
        __syncthreads();
        decode(g1, 1);
        __syncthreads();
        compute(1);
    }

    // Epilogue: each wave stages 32 output rows at a time through LDS (fp32,
    // alpha applied) and writes them back as 16-byte row segments.
    const float alpha = (1.0f / *a_senc) * (1.0f / *b_senc);
    const int64_t m0 = tile_m * kBM + wm * 128, n0 = tile_n * kBN + wn * 64;
    constexpr int kEpiStride = 68;   // floats per staged row (64 + 4 pad)
    __syncthreads();                 // every wave is done reading the operand stages
    float* stage_out = reinterpret_cast<float*>(&lds[0][0][0]) + wave * 32 * kEpiStride;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = (e >> 2) * 8 + g * 4 + (e & 3);
                stage_out[r * kEpiStride + 32 * tn + lr] = acc[tm][tn][e] * alpha;
            }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        // 32 rows x 64 columns = 32 x 16 float4; lane handles float4 (row, q)
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int idx = it * 64 + lane;
            const int r = idx >> 4, q = idx & 15;
            const float4 v = *reinterpret_cast<const float4*>(stage_out + r * kEpiStride + 4 * q);
            const int64_t row = m0 + 32 * tm + r, col = n0 + 4 * q;
            if (row < M && col < N) {
                if constexpr (kOutF32) {
                    float* dst = static_cast<float*>(c) + row * ldc + col;
                    if (col + 4 <= N) {
                        *reinterpret_cast<float4*>(dst) = v;
                    } else {
                        dst[0] = v.x;
                        if (col + 1 < N) dst[1] = v.y;
                        if (col + 2 < N) dst[2] = v.z;
                    }
                } else {
                    uint16_t* dst = static_cast<uint16_t*>(c) + row * ldc + col;
                    const uint16_t b0 = f32_to_bf16_rne(v.x), b1 = f32_to_bf16_rne(v.y);
                    const uint16_t b2 = f32_to_bf16_rne(v.z), b3 = f32_to_bf16_rne(v.w);
                    if (col + 4 <= N) {
                        *reinterpret_cast<uint2*>(dst) =
                            make_uint2(b0 | ((uint32_t)b1 << 16), b2 | ((uint32_t)b3 << 16));
                    } else {
                        dst[0] = b0;
                        if (col + 1 < N) dst[1] = b1;
                        if (col + 2 < N) dst[2] = b2;
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
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
        hipLaunchKernelGGL(k_gemm_nt<true>, grid, dim3(512), 0, s, a.codes, a.ld_codes, a.scales,
                           a.ld_scales, a.scale_row_shift, a.s_enc, b.codes, b.ld_codes, b.scales,
                           b.ld_scales, b.scale_row_shift, b.s_enc, M, N, K, c, ldc);
    else
        hipLaunchKernelGGL(k_gemm_nt<false>, grid, dim3(512), 0, s, a.codes, a.ld_codes, a.scales,
                           a.ld_scales, a.scale_row_shift, a.s_enc, b.codes, b.ld_codes, b.scales,
                           b.ld_scales, b.scale_row_shift, b.s_enc, M, N, K, c, ldc);
}

}  // namespace nvfp4
