// gemm.hip -- GEMMs on gfx950 matrix cores: over NVFP4 operands, and over
// bf16 operands for the layers that stay in high precision.
//
// Passes: "Pretraining Large Language Models with NVFP4" (gist.science
// summary), Technische Zusammenfassung 2.B.2 (Fprop, Dgrad, Wgrad GEMMs of a
// linear layer); format 2.A (E2M1 codes, E4M3 scale per 16 elements, FP32
// tensor scale); 2.B.1 (a few layers keep BF16).
//
// Both kernels compute C[m, n] = alpha sum_k A[m, k] B[n, k] with a
// workgroup of 8 waves (two per SIMD) per 256x256 output tile, in K steps of
// 64, and 4x2 MFMA 32x32x16 tiles per wave (a 128x64 slab, 128 fp32
// accumulators).  Two LDS stages alternate: while the MFMAs consume one, the
// next step is written into the other.  Workgroups are renumbered so that
// each XCD gets a contiguous range of tiles, walked in groups of 8 tile rows
// so that concurrently running tiles share operand panels.  The epilogue
// stages 32 output rows per wave through LDS and stores 16-byte row segments.
//
// NVFP4 (k_gemm_nv).  The pages' GEMM runs on Blackwell FP4 tensor cores;
// gfx950's block-scaled FP4 MFMA takes power-of-two scales per 32 elements,
// which cannot express an E4M3 scale per 16 elements.  Here every element is
// decoded to the exact fp16 value q * S_b (E2M1 times E4M3 needs at most 6
// significant bits and lies in [2^-10, 2688], inside fp16's normal range):
// the hardware converts a byte of two codes to an fp16 pair, and one packed
// fp16 multiply applies the block scale.  The fp16 MFMA accumulates exact
// products in fp32, and the epilogue multiplies by
// alpha = (1/s_enc_a) (1/s_enc_b), kept apart from its exponent when it falls
// below fp32's normal range (output_scale).  The A tile (shared by 4 waves) is
// decoded once per workgroup into fp16 LDS rows; the B tile (shared by 2
// waves) stays raw in LDS -- 48 bytes per row instead of 144 -- and each
// wave decodes its own B fragments after reading them, trading a little
// VALU work for a third less LDS traffic, the resource that bounds this
// loop.  Each thread loads half an A row and half a B row per step, and
// the scales of its rows three steps at a time; the loads run three steps
// ahead of the MFMAs in three register stages.  The epilogue converts to
// bf16 with the packed hardware conversion.
// NVFP4 operands are "rows x K" with K contiguous (the dgrad weight operand
// is the transposed 16x16-block copy written by the quantiser).
//
// bf16 (k_gemm_bf16).  A bf16 operand is either "rows x K" (layout N) or
// "K x rows" (layout T, rows contiguous), so the three bf16 passes read X,
// W and dY where they lie.  Per step each thread moves 8 pieces of 16 bytes
// into LDS, where a layout-T tile stays K-major and its MFMA fragments come
// from gfx950's transposing LDS reads; the loads run one step ahead.
//
// Also here: the MXFP4 comparison GEMM (k_gemm_mx, block-scaled FP4 MFMA),
// the reduce of the tail-split launches (k_splitk_reduce), and a
// register-only stream of the matrix instructions (k_mfma_sustain) that the
// bench times for the throughput the chip sustains under load.
//
// Lane layout of v_mfma_f32_32x32x16_{f16,bf16}: lane l supplies row (A) or
// column (B) l % 32 and 8 consecutive k (the "half" l / 32 of the 16-wide
// step); accumulator j of lane l is row (j/4)*8 + (l/32)*4 + j%4, column l % 32.
#include <type_traits>
#include <utility>

#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kBM = 256, kBN = 256, kKS = 64;  // workgroup tile and K step
constexpr int kRowBytes = 144;                 // LDS row: 64 16-bit values (128 B) + 16 B pad
constexpr int kOpBytes = 256 * kRowBytes;      // one 16-bit operand tile, one stage
constexpr int kEpiStride = 68;                 // floats per staged output row (64 + 4 pad)

// Kernel arguments of one operand; fields a kernel does not use stay zero.
struct OpArgs {
    const void* data;       // NVFP4 codes, or bf16 values
    int64_t ld;             // bytes (codes) or elements (bf16) between consecutive rows in memory
    const uint8_t* scales;  // NVFP4: E4M3 block scales
    int64_t ld_scales;
    int scale_shift;        // NVFP4: scale row = row >> scale_shift
    const float* s_enc;     // NVFP4: tensor encode scale
    int64_t kst;            // NVFP4: code bytes from one 64-element K step of a row to the next
    bool il;                // NVFP4: codes 4-row interleaved (code_offset)
};

// The kernel arguments of an NVFP4 operand of k_gemm_nv.
OpArgs nv_args(const GemmOperand& g)
{
    return OpArgs{g.codes, g.ld_codes, g.scales, g.ld_scales, g.scale_row_shift, g.s_enc,
                  g.il ? 128 : 32, g.il};
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Two fp32 values -> two bf16 (round to nearest even), a in the low half:
// one v_cvt_pk_bf16_f32.  An exhaustive in-bounds probe over every non-NaN
// fp32 bit pattern (subnormals and infinities included) found it equal to
// f32_to_bf16_rne; the outputs here are never NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

// This workgroup's output tile.  Workgroups are dealt round-robin to the 8
// XCDs; renumbering gives each XCD a contiguous range, walked in groups of 8
// tile rows, column by column.
template <int kTM = kBM>
__device__ __forceinline__ void tile_of(int64_t M, int64_t N, int64_t& tile_m, int64_t& tile_n,
                                        int64_t hw = -1)
{
    const int64_t tiles_m = (M + kTM - 1) / kTM, tiles_n = (N + kBN - 1) / kBN;
    const int64_t T = tiles_m * tiles_n;
    if (hw < 0) hw = blockIdx.x;
    const int64_t L = (T % 8 == 0) ? (hw % 8) * (T / 8) + hw / 8 : hw;
    const int64_t GM = 8;
    const int64_t group = L / (GM * tiles_n);
    const int64_t first_m = group * GM;
    const int64_t gsz = (tiles_m - first_m < GM) ? (tiles_m - first_m) : GM;
    const int64_t in_group = L - group * GM * tiles_n;
    tile_m = first_m + in_group % gsz;
    tile_n = in_group / gsz;
}

// Epilogue: each wave stages its output rows through its own LDS area
// `stage_out` (32 x kEpiStride floats; every wave must be done with the
// operand stages) and writes them back as 16-byte row segments: fp32 values
// (alpha applied) 32 rows at a time, or for a bf16 output without maxima
// the rounded bf16 values 64 rows at a time.
//
// kAmax (bf16 output only) also folds the output into the tensor maxima its
// next quantisation needs: 1 = max |y| over the bf16 values (into
// amax_bits[0]); 2 = that and the max over the 16-point RHT, along the rows
// (tokens), of every aligned 16-row chunk of a column (into amax_rht_bits[0];
// M a multiple of 16).  The values are rounded to bf16 before they are
// staged, so both maxima see exactly the stored tensor; they go out as uint
// bits of non-negative floats through one atomic max per wave.
//
// The transform runs on the accumulator registers.  In the 32 x 32 MFMA
// result a lane holds column lr of row 8 (e / 4) + 4 g + e % 4, so a 16-row
// chunk of a column is split between lanes lr and lr + 32 (row bit 2 = g),
// 8 values each: row bits 0, 1 are bits 0, 1 of e and row bit 3 is bit 2.
// Strides 1 and 2 run in each lane; then v_permlane32_swap trades the
// column-tn = 0 values of lanes 32-63 for the column-tn = 1 values of lanes
// 0-31, so every lane holds one whole chunk (lane l: column l of the 64) and runs
// strides 4 and 8 -- the butterfly order of the transform, so the fp32
// values are the ones a separate pass computes.
template <bool kOutF32, int kAmax = 0>
__device__ __forceinline__ void store_tile(const float16_t (&acc)[4][2], float alpha,
                                           float* stage_out, int64_t m0, int64_t n0, int64_t M,
                                           int64_t N, void* __restrict__ c, int64_t ldc,
                                           uint32_t* amax_bits = nullptr,
                                           uint32_t* amax_rht_bits = nullptr, uint32_t mask = 0u)
{
    static_assert(kAmax == 0 || !kOutF32, "output maxima are taken of bf16 outputs");
    const int lane = threadIdx.x & 63;
    const int g = lane >> 5, lr = lane & 31;
    if constexpr (!kOutF32 && kAmax == 0) {
        // bf16 output without maxima: the values are rounded before they are
        // staged, so a round holds 64 rows x 64 columns (128-byte rows, 8 KB,
        // inside the wave's 32 x kEpiStride floats) and leaves as 16-byte row
        // pieces: half the rounds, LDS reads and stores of fp32 staging
        // (fprop +1.0 %, dgrad +0.3 %, bit-identical)
        constexpr int kP = 64;
        static_assert(64 * kP * 2 <= 32 * kEpiStride * 4, "the bf16 rows fit the wave's staging area");
        uint16_t* st = reinterpret_cast<uint16_t*>(stage_out);
        const bool al16 = ((reinterpret_cast<uintptr_t>(c) & 15) == 0) && ((ldc & 7) == 0);
#pragma unroll
        for (int R = 0; R < 2; ++R) {
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                const int tm = 2 * R + t2;
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                    for (int e = 0; e < 16; e += 2) {
                        const int r = 32 * t2 + (e >> 2) * 8 + g * 4 + (e & 3);
                        const uint32_t p = bf16x2_rne(acc[tm][tn][e] * alpha, acc[tm][tn][e + 1] * alpha);
                        st[r * kP + 32 * tn + lr] = (uint16_t)p;
                        st[(r + 1) * kP + 32 * tn + lr] = (uint16_t)(p >> 16);
                    }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int idx = it * 64 + lane;
                const int r = idx >> 3, q = idx & 7;
                const uint4 v = *reinterpret_cast<const uint4*>(st + r * kP + 8 * q);
                const int64_t row = m0 + 64 * R + r, col = n0 + 8 * q;
                if (row < M && col < N) {
                    uint16_t* dst = static_cast<uint16_t*>(c) + row * ldc + col;
                    if (col + 8 <= N && al16) {  // streaming store: the output is not read back here
                        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
                        __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(dst));
                    } else {
                        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            if (col + k < N) dst[k] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        return;
    }
    uint32_t am = 0u;  // max |y| as float bits (magnitudes compare as integers)
    float rm = 0.0f;   // max |unscaled transform|
    const bool inside = m0 + 128 <= M && n0 + 64 <= N;  // the wave's whole slab is stored
    uint32_t sgn[8];  // sign bit of row 8 (k / 4) + 4 g + k % 4 of a chunk
    if constexpr (kAmax == 2) {
        const uint32_t mg = g ? (mask >> 4) : mask;
#pragma unroll
        for (int k = 0; k < 8; ++k) sgn[k] = ((mg >> ((k >> 2) * 8 + (k & 3))) & 1u) << 31;
    }
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        float y[2][16];
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = (e >> 2) * 8 + g * 4 + (e & 3);
                float v = acc[tm][tn][e] * alpha;
                if constexpr (kAmax > 0) v = __uint_as_float(bf16x2_rne(v, v) << 16);
                y[tn][e] = v;
                stage_out[r * kEpiStride + 32 * tn + lr] = v;
            }
        if constexpr (kAmax > 0) {
            if (inside) {
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        am = max(am, __float_as_uint(y[tn][e]) & 0x7FFFFFFFu);
            } else {
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int64_t row = m0 + 32 * tm + (e >> 2) * 8 + g * 4 + (e & 3);
                        if (row < M && n0 + 32 * tn + lr < N)
                            am = max(am, __float_as_uint(y[tn][e]) & 0x7FFFFFFFu);
                    }
            }
        }
        if constexpr (kAmax == 2) {
#pragma unroll
            for (int ch = 0; ch < 2; ++ch) {
                float h[2][8];
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) {
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        h[tn][k] = __uint_as_float(__float_as_uint(y[tn][8 * ch + k]) ^ sgn[k]);
#pragma unroll
                    for (int st = 1; st <= 2; st <<= 1)
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            if ((k & st) == 0) {
                                const float a = h[tn][k], b = h[tn][k + st];
                                h[tn][k] = a + b;
                                h[tn][k + st] = a - b;
                            }
                }
                float lo[8], hi[8];  // the chunk's rows with bit 2 clear / set
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(h[0][k]),
                                                                    __float_as_uint(h[1][k]),
                                                                    false, false);
                    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
                    lo[k] = a + b;  // stride 4
                    hi[k] = a - b;
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {  // stride 8
                    const float a = lo[k], b = lo[k + 4], c2 = hi[k], d = hi[k + 4];
                    lo[k] = a + b;
                    lo[k + 4] = a - b;
                    hi[k] = c2 + d;
                    hi[k + 4] = c2 - d;
                }
                if (n0 + lane < N && m0 + 32 * tm + 16 * ch < M)
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        rm = __builtin_fmaxf(rm, __builtin_fmaxf(__builtin_fabsf(lo[k]),
                                                                 __builtin_fabsf(hi[k])));
            }
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
                    if (col + 4 <= N) {  // streaming store: the output is not read back here
                        typedef float f32x4_t __attribute__((ext_vector_type(4)));
                        __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t*>(dst));
                    } else {
                        dst[0] = v.x;
                        if (col + 1 < N) dst[1] = v.y;
                        if (col + 2 < N) dst[2] = v.z;
                    }
                } else {
                    uint16_t* dst = static_cast<uint16_t*>(c) + row * ldc + col;
                    uint32_t w01, w23;  // bf16 pairs (columns col, col + 1 and col + 2, col + 3)
                    if constexpr (kAmax > 0) {  // staged values are bf16 already
                        w01 = __builtin_amdgcn_perm(__float_as_uint(v.y), __float_as_uint(v.x), 0x07060302u);
                        w23 = __builtin_amdgcn_perm(__float_as_uint(v.w), __float_as_uint(v.z), 0x07060302u);
                    } else {
                        w01 = bf16x2_rne(v.x, v.y);
                        w23 = bf16x2_rne(v.z, v.w);
                    }
                    if (col + 4 <= N) {  // streaming store, as above
                        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                        __builtin_nontemporal_store(u32x2_t{w01, w23}, reinterpret_cast<u32x2_t*>(dst));
                    } else {
                        dst[0] = (uint16_t)w01;
                        if (col + 1 < N) dst[1] = (uint16_t)(w01 >> 16);
                        if (col + 2 < N) dst[2] = (uint16_t)w23;
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    if constexpr (kAmax > 0) {
        const uint32_t ab = wave_max_u32(am);
        if (lane == 0) atomicMax(amax_bits, ab);
        if constexpr (kAmax == 2) {
            // rounding is monotonic: the max of the scaled values is the scaled max
            const uint32_t rb = wave_max_u32(__float_as_uint(rm * 0.25f));
            if (lane == 0) atomicMax(amax_rht_bits, rb);
        }
    }
}

__device__ __forceinline__ void zero_acc(float16_t (&acc)[4][2])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
}

// 8 E2M1 codes (one dword, low nibble first) times the fp16 block scale S
// (broadcast pair): the exact fp16 values, in code order.
__device__ __forceinline__ half8_t decode8(uint32_t w, half2_t S)
{
    const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * S;
    const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * S;
    const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * S;
    const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * S;
    return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                   __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5,
                                   6, 7);
}

// ---------------------------------------------------------------------------
// NVFP4 x NVFP4
//
// LDS stage: A as fp16 rows (256 x 144 B), B as raw codes (256 x 48 B: 32
// code bytes + pad, so that 16-byte reads of 8 consecutive rows hit distinct
// banks) and B scales (256 x 4 B).  Thread t handles half h = t % 2 of tile
// row t / 2 of both operands: 16 code bytes (32 k, blocks 2h and 2h+1) and 2
// scale bytes each.
//
// Within a step the MFMA sub-steps take the k in a permuted order (the
// contraction does not depend on it): lane half g of sub-step i covers
// k = 32 g + 8 i .. +7.  A lane's B fragments for the whole step are then 16
// contiguous code bytes -- one 16-byte LDS read -- and sub-step i uses block
// 2g + i/2; the A fragments are read from the matching fp16 offsets.
// ---------------------------------------------------------------------------

constexpr int kBRow = 48;
constexpr int kBOp = 256 * kBRow;

// LDS bytes of one stage of a tile with kTM rows of A: A decoded (kTM x
// 144 B), B raw (256 x 48 B), B scales (256 x 4 B).
template <int kTM>
constexpr int nv_stage_bytes() { return kTM * kRowBytes + kBOp + 256 * 4; }

// One thread's share of a K step: half an A row, and kRB half B rows
// (kRB = 1 for 256-row tiles of 512 threads, 2 for 128-row tiles of 256).
template <int kRB>
struct NvRow {
    uint4 ca, cb[kRB];      // 16 code bytes of its A and B half rows
    uint32_t sa, sb[kRB];   // its 2 A and 2 B scale bytes per half row, as loaded
};

}  // namespace

// kTM = 256: 8 waves (2 x 4, each a 128 x 64 slab), one workgroup per CU.
// kTM = 128: 4 waves (1 x 4), 62 KB of LDS, two workgroups per CU -- their
// phases drift apart, so one workgroup's stores, barriers and epilogue run
// while the other's waves issue MFMAs.
// Split tail (split > 1): workgroups past `full_tiles` take the remaining
// tiles `split` ways along K, in whole K steps (the partial last step in the
// last part), and store their raw fp32 sums (no output scale) into `ws`, one
// 256 x 256 row-major tile per part; k_splitk_reduce then adds the parts in
// order and writes the output.  The launch then fills the last, otherwise
// partial, wave of tiles with parts of equal length.
template <int kTM, bool kOutF32, int kAmax = 0>
__global__ __launch_bounds__(2 * kTM, 256 / kTM) void k_gemm_nv(OpArgs A, OpArgs B, int64_t M, int64_t N,
                                                    int64_t K, void* __restrict__ c, int64_t ldc,
                                                    uint32_t* amax_bits = nullptr,
                                                    uint32_t* amax_rht_bits = nullptr,
                                                    uint32_t mask = 0u, int64_t full_tiles = 0,
                                                    int split = 1, float* __restrict__ ws = nullptr)
{
    constexpr int kRB = 256 / kTM;
    constexpr int kAOp = kTM * kRowBytes;
    constexpr int kStage = nv_stage_bytes<kTM>();
    static_assert((2 * kTM / 64) * 32 * kEpiStride * 4 <= 2 * kStage, "epilogue rows fit the stages");
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, lr = lane & 31;
    int64_t hw = blockIdx.x, part = 0;
    if (split > 1 && hw >= full_tiles) {
        part = (hw - full_tiles) % split;
        hw = full_tiles + (hw - full_tiles) / split;
    }
    int64_t tile_m, tile_n;
    tile_of<kTM>(M, N, tile_m, tile_n, hw);
    if (split > 1 && hw >= full_tiles) {  // this part's K steps [s0, s1)
        const int64_t nst = (K + kKS - 1) / kKS;
        const int64_t s0 = nst * part / split, s1 = nst * (part + 1) / split;
        const int64_t k0 = s0 * kKS, k1 = s1 * kKS < K ? s1 * kKS : K;
        A.data = static_cast<const uint8_t*>(A.data) + s0 * A.kst;
        B.data = static_cast<const uint8_t*>(B.data) + s0 * B.kst;
        A.scales += k0 >> 4;
        B.scales += k0 >> 4;
        K = k1 - k0;
    }

    // half h of tile row `row` of A and of tile rows row + kTM j of B (rows
    // past the operand re-read its last row; they are never stored)
    const int row = tid >> 1, h = tid & 1;
    int64_t ra = tile_m * kTM + row;
    ra = ra < M ? ra : M - 1;
    // Addresses are a uniform base (SGPRs; the K offset of a step is added
    // there) plus a 32-bit per-thread byte offset: an operand's codes and
    // scales each span less than 4 GiB (the ABI checks it).
    const uint8_t* const Ad = static_cast<const uint8_t*>(A.data);
    const uint8_t* const Bd = static_cast<const uint8_t*>(B.data);
    const uint32_t oa = (uint32_t)code_offset(ra, 16 * h, A.ld, A.il);  // codes of the half row
    const uint32_t qa = (uint32_t)((ra >> A.scale_shift) * A.ld_scales);  // the row's scales
    uint32_t ob[kRB], qb[kRB];
#pragma unroll
    for (int j = 0; j < kRB; ++j) {
        int64_t rb = tile_n * kBN + row + kTM * j;
        rb = rb < N ? rb : N - 1;
        ob[j] = (uint32_t)code_offset(rb, 16 * h, B.ld, B.il);
        qb[j] = (uint32_t)((rb >> B.scale_shift) * B.ld_scales);
    }
    const int64_t nblk = K >> 4;

    auto load_full = [&](int64_t k0, NvRow<kRB>& w) {
        w.ca = *reinterpret_cast<const uint4*>(Ad + (k0 >> 6) * A.kst + oa);
#pragma unroll
        for (int j = 0; j < kRB; ++j) w.cb[j] = *reinterpret_cast<const uint4*>(Bd + (k0 >> 6) * B.kst + ob[j]);
        w.sa = *reinterpret_cast<const uint16_t*>(A.scales + (k0 >> 4) + (qa + 2u * h));
#pragma unroll
        for (int j = 0; j < kRB; ++j)
            w.sb[j] = *reinterpret_cast<const uint16_t*>(B.scales + (k0 >> 4) + (qb[j] + 2u * h));
    };
    // partial last step: blocks past K get zero scales, so their codes decode
    // to zero (the 16 code bytes of a half row with one valid block still lie
    // inside the row, whose length is rounded up to 32 codes)
    auto load_tail = [&](int64_t k0, NvRow<kRB>& w) {
        const int64_t b0 = (k0 >> 4) + 2 * h;
        w.ca = b0 < nblk ? *reinterpret_cast<const uint4*>(Ad + (k0 >> 6) * A.kst + oa) : make_uint4(0, 0, 0, 0);
        uint32_t sa = 0u;
        for (int i = 0; i < 2; ++i)
            if (b0 + i < nblk) sa |= (uint32_t)A.scales[b0 + i + qa] << (8 * i);
        w.sa = sa;
#pragma unroll
        for (int j = 0; j < kRB; ++j) {
            w.cb[j] = b0 < nblk ? *reinterpret_cast<const uint4*>(Bd + (k0 >> 6) * B.kst + ob[j]) : make_uint4(0, 0, 0, 0);
            uint32_t sb = 0u;
            for (int i = 0; i < 2; ++i)
                if (b0 + i < nblk) sb |= (uint32_t)B.scales[b0 + i + qb[j]] << (8 * i);
            w.sb[j] = sb;
        }
    };
    // A half row decoded to fp16 q * S in natural k order; B half rows stored
    // raw.  Scale words: bits [sh, sh + 16) of sa (and of each sb) are the
    // half row's two scale bytes.  kPin: the words come from a load of three
    // steps' scales; an empty asm keeps their shifts here (hoisted next to
    // that load, a shift would wait for the loads issued with it).
    auto put_s = [&](auto pin, const NvRow<kRB>& w, int st, uint32_t sa, const uint32_t (&sbw)[kRB], int sh) {
        constexpr bool kPin = decltype(pin)::value;
        uint32_t sb[kRB];
#pragma unroll
        for (int j = 0; j < kRB; ++j) sb[j] = sbw[j];
        if constexpr (kPin) {
            asm volatile("" : "+v"(sa));
#pragma unroll
            for (int j = 0; j < kRB; ++j) asm volatile("" : "+v"(sb[j]));
        }
        uint8_t* base = lds + st * kStage;
        const half2_t pair = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa >> sh, 1.0f, false);
        const half2_t S0 = __builtin_shufflevector(pair, pair, 0, 0);
        const half2_t S1 = __builtin_shufflevector(pair, pair, 1, 1);
        const uint32_t cw[4] = {w.ca.x, w.ca.y, w.ca.z, w.ca.w};
#pragma unroll
        for (int d = 0; d < 4; ++d)  // dword d: k 32h + 8d .. +7, block 2h + d/2
            *reinterpret_cast<half8_t*>(base + row * kRowBytes + 64 * h + 16 * d) =
                decode8(cw[d], d < 2 ? S0 : S1);
#pragma unroll
        for (int j = 0; j < kRB; ++j) {
            *reinterpret_cast<uint4*>(base + kAOp + (row + kTM * j) * kBRow + 16 * h) = w.cb[j];
            *reinterpret_cast<uint16_t*>(base + kAOp + kBOp + (row + kTM * j) * 4 + 2 * h) = (uint16_t)(sb[j] >> sh);
        }
    };
    auto put = [&](const NvRow<kRB>& w, int st) { put_s(std::false_type{}, w, st, w.sa, w.sb, 0); };

    float16_t acc[4][2];
    zero_acc(acc);
    const int wm = wave >> 2, wn = wave & 3;
    const int a_frag = (wm * 128 + lr) * kRowBytes + 64 * g;  // + 32 tm rows, + 16 i bytes
    const int b_row = wn * 64 + lr;                           // + 32 tn

    auto compute = [&](int st) {
        const uint8_t* As = lds + st * kStage;
        const uint8_t* Bs = As + kAOp;
        const uint8_t* Bsc = Bs + kBOp;
        uint4 bc[2];
        half2_t bpair[2];
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
            bc[tn] = *reinterpret_cast<const uint4*>(Bs + (b_row + 32 * tn) * kBRow + 16 * g);
            // this lane's blocks 2g and 2g+1, moved to the low half
            const uint32_t sw = *reinterpret_cast<const uint32_t*>(Bsc + (b_row + 32 * tn) * 4) >> (16 * g);
            bpair[tn] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
        }
        half8_t af[2][4];  // A fragments of two sub-steps in flight
#pragma unroll
        for (int t = 0; t < 4; ++t) af[0][t] = *reinterpret_cast<const half8_t*>(As + a_frag + t * 32 * kRowBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cur = i & 1, nxt = cur ^ 1;
            if (i < 3) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    af[nxt][t] = *reinterpret_cast<const half8_t*>(As + a_frag + t * 32 * kRowBytes + 16 * (i + 1));
            }
            half8_t bf[2];
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) {
                const half2_t S = (i < 2) ? __builtin_shufflevector(bpair[tn], bpair[tn], 0, 0)
                                          : __builtin_shufflevector(bpair[tn], bpair[tn], 1, 1);
                const uint32_t w = i == 0 ? bc[tn].x : i == 1 ? bc[tn].y : i == 2 ? bc[tn].z : bc[tn].w;
                bf[tn] = decode8(w, S);
            }
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[cur][tm], bf[tn], acc[tm][tn], 0, 0, 0);
        }
        // Issue order of the LDS reads and MFMAs: the B words, B scales and
        // the A fragments of sub-steps 0 and 1 first, then each sub-step's 8
        // MFMAs followed by the A reads of the sub-step after next, so every
        // fragment is read a whole sub-step (8 MFMAs) before its use.  Left
        // to itself the scheduler issues each read two MFMAs ahead to save
        // registers, which exposes the LDS latency.
        __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // 12 LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // sub-step 0
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // A of sub-step 2
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // sub-step 1
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // A of sub-step 3
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // sub-steps 2, 3
    };

    // Step t's rows live in register stage t % 3 and its tile in LDS stage
    // t % 2.  Loads are unconditional (clamped to the last full step) so the
    // compiler's wait counts stay exact.
    const int64_t nsteps = (K + kKS - 1) / kKS;
    const int64_t nfull = K / kKS;
    int64_t s = 0;
    NvRow<kRB> g0, g1, g2;
    if (nfull > 0) {
        load_full(0, g0);
        load_full((nfull > 1 ? 1 : 0) * kKS, g1);
        load_full((nfull > 2 ? 2 : nfull - 1) * kKS, g2);
        put(g0, 0);
    }
    __syncthreads();
    auto step = [&](auto c3, int64_t t) {
        constexpr int r = decltype(c3)::value;
        const int st = (int)(t & 1);
        NvRow<kRB>& done = r == 0 ? g0 : (r == 1 ? g1 : g2);  // step t, already in LDS
        NvRow<kRB>& next = r == 0 ? g1 : (r == 1 ? g2 : g0);  // step t + 1
        load_full((t + 3 < nfull ? t + 3 : nfull - 1) * kKS, done);
        compute(st);
        put(next, st ^ 1);  // past the last full step: harmless, never read
        __syncthreads();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // Scale loads three steps at a time.  A step needs 4 scale bytes of a
    // row; a 2-byte load per thread, operand and step costs the memory
    // pipeline as much as a 16-byte code load (both touch one cache line per
    // row), so while whole steps remain, one 12-byte load (4-byte aligned:
    // the ABI requires it of scale rows) brings the scales of three steps.
    // Register sets P and Q alternate: on entry to a 6-step round P holds
    // steps s .. s+2; Q is loaded with s+3 .. s+5 at step s, P with
    // s+6 .. s+8 at step s+3.
    if (nfull >= 9) {
        uint3 Pa = *reinterpret_cast<const uint3*>(A.scales + qa), Qa;
        uint3 Pb[kRB], Qb[kRB];
#pragma unroll
        for (int j = 0; j < kRB; ++j) Pb[j] = *reinterpret_cast<const uint3*>(B.scales + qb[j]);
        const int sh = 16 * h;
        auto gstep = [&](auto c6, int64_t t, uint3& Ca, uint3 (&Cb)[kRB], uint3& Na, uint3 (&Nb)[kRB]) {
            constexpr int r = decltype(c6)::value % 3;
            const int st = (int)(t & 1);
            NvRow<kRB>& done = r == 0 ? g0 : (r == 1 ? g1 : g2);  // step t, already in LDS
            NvRow<kRB>& next = r == 0 ? g1 : (r == 1 ? g2 : g0);  // step t + 1
            const int64_t k3 = (t + 3) * kKS;  // a whole step: t + 3 < nfull
            done.ca = *reinterpret_cast<const uint4*>(Ad + (k3 >> 6) * A.kst + oa);
#pragma unroll
            for (int j = 0; j < kRB; ++j) done.cb[j] = *reinterpret_cast<const uint4*>(Bd + (k3 >> 6) * B.kst + ob[j]);
            if constexpr (r == 0) {
                Na = *reinterpret_cast<const uint3*>(A.scales + 4 * (t + 3) + qa);
#pragma unroll
                for (int j = 0; j < kRB; ++j) Nb[j] = *reinterpret_cast<const uint3*>(B.scales + 4 * (t + 3) + qb[j]);
            }
            compute(st);
            uint32_t wb[kRB];
#pragma unroll
            for (int j = 0; j < kRB; ++j) wb[j] = r == 0 ? Cb[j].y : (r == 1 ? Cb[j].z : Nb[j].x);
            put_s(std::true_type{}, next, st ^ 1, r == 0 ? Ca.y : (r == 1 ? Ca.z : Na.x), wb, sh);
            __syncthreads();
        };
        using I3 = std::integral_constant<int, 3>;
        using I4 = std::integral_constant<int, 4>;
        using I5 = std::integral_constant<int, 5>;
        for (; s + 9 <= nfull; s += 6) {
            gstep(I0{}, s, Pa, Pb, Qa, Qb);
            gstep(I1{}, s + 1, Pa, Pb, Qa, Qb);
            gstep(I2{}, s + 2, Pa, Pb, Qa, Qb);
            gstep(I3{}, s + 3, Qa, Qb, Pa, Pb);
            gstep(I4{}, s + 4, Qa, Qb, Pa, Pb);
            gstep(I5{}, s + 5, Qa, Qb, Pa, Pb);
        }
        // steps s+1, s+2 (in flight) continue with one scale load per step
        g1.sa = Pa.y >> sh;
        g2.sa = Pa.z >> sh;
#pragma unroll
        for (int j = 0; j < kRB; ++j) {
            g1.sb[j] = Pb[j].y >> sh;
            g2.sb[j] = Pb[j].z >> sh;
        }
    }
    for (; s + 3 <= nfull; s += 3) {
        step(I0{}, s);
        step(I1{}, s + 1);
        step(I2{}, s + 2);
    }
    if (s < nfull) step(I0{}, s++);
    if (s < nfull) step(I1{}, s++);
    if (nfull < nsteps) {  // partial last step, into LDS stage nfull % 2
        load_tail(nfull * kKS, g0);
        put(g0, (int)(nfull & 1));
        __syncthreads();
        compute((int)(nfull & 1));
    }

    if (split > 1 && hw >= full_tiles) {  // one part of a split tile: raw sums into ws
        float* dst = ws + ((hw - full_tiles) * split + part) * (int64_t)(kTM * kBN);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = wm * 128 + tm * 32 + (e >> 2) * 8 + g * 4 + (e & 3);
                    __builtin_nontemporal_store(acc[tm][tn][e], dst + r * kBN + wn * 64 + tn * 32 + lr);
                }
        return;
    }
    float alpha;
    int alpha_exp;
    output_scale(*A.s_enc, *B.s_enc, alpha, alpha_exp);
    if (alpha_exp != 0) {  // (uniform) output scale below fp32's normal range
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = __builtin_ldexpf(acc[i][j][e] * alpha, alpha_exp);
        alpha = 1.0f;
    }
    __syncthreads();  // every wave is done reading the operand stages
    store_tile<kOutF32, kAmax>(acc, alpha, reinterpret_cast<float*>(lds) + wave * 32 * kEpiStride,
                               tile_m * kTM + wm * 128, tile_n * kBN + wn * 64, M, N, c, ldc,
                               amax_bits, amax_rht_bits, mask);
}

namespace {

// ---------------------------------------------------------------------------
// MXFP4 x MXFP4 -- the format NVFP4 is compared with (32-element blocks, one
// UE8M0 power-of-two scale each, no tensor scale).
//
// gfx950's block-scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 with FP4
// operands reads E2M1 codes directly with one E8M0 scale per lane: lane l
// supplies row (A) or column (B) l % 32 and the 32 consecutive k of half
// l / 32 of its 64-wide step -- exactly one MX block, 16 code bytes -- so the
// operands enter the matrix cores as stored, with no decode.  Same tile,
// wave grid and epilogue as k_gemm_nv; a K step is 128 (4 blocks, 64 code
// bytes per row) in two MFMA sub-steps of 64, and a wave reads all its
// fragments of a step before its first MFMA.
//
// No VGPR staging: the operands move from global memory straight into LDS
// (global_load_lds_dwordx4, 16 bytes per lane, 1 KB per wave instruction
// landing contiguously), three stages deep, two steps ahead.  Rows are 64
// packed bytes; chunk c of row r sits at position c ^ swz(r) so that the
// fragment reads (16 bytes of 16 consecutive rows) hit distinct banks.  Each
// stage is its own array so that the compiler can tell that the loads in
// flight never write the stage being read, and the steady-state barrier
// carries no release fence, whose wait for every outstanding load would
// empty the pipeline; the waits on the loads are the explicit vmcnt.
// ---------------------------------------------------------------------------

constexpr int kMxKS = 128;
constexpr int kMxA = 0, kMxB = 16384, kMxS = 32768;  // codes of A, B; scales (A, then B)
constexpr int kMxStage = kMxS + 2048;
static_assert(4 * 32 * kEpiStride * 4 <= kMxStage, "four waves' epilogue rows fit one stage");

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ v8i_t mx_frag(const uint8_t* p)
{
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(p);
    return v8i_t{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
}

__device__ __forceinline__ int mx_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

}  // namespace

template <bool kOutF32>
__global__ __launch_bounds__(512, 1) void k_gemm_mx(OpArgs A, OpArgs B, int64_t M, int64_t N,
                                                    int64_t K, void* __restrict__ c, int64_t ldc)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds0[kMxStage];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[kMxStage];
    __shared__ __attribute__((aligned(16))) uint8_t lds2[kMxStage];
    // scales of three steps (12 bytes per row; A rows, then B rows), two sets;
    // a 12-byte LDS load lands each lane's bytes 16 bytes apart
    __shared__ __attribute__((aligned(16))) uint8_t sg0[2 * 256 * 16];
    __shared__ __attribute__((aligned(16))) uint8_t sg1[2 * 256 * 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, lr = lane & 31;
    int64_t tile_m, tile_n;
    tile_of(M, N, tile_m, tile_n);
    const int64_t nblk = K >> 5;

    // Load plan: wave w moves code pieces q = 4w .. 4w+3 (piece q: operand
    // q / 16, tile rows 16 (q % 16) + lane / 4; lane % 4 is the chunk
    // position in LDS, holding chunk (lane % 4) ^ swz(row) of the row) and
    // one scale piece (rows 64 (w % 4) + lane, 4 bytes).  Waves 0-3 move A,
    // waves 4-7 move B, so every base pointer is wave-uniform; rows past the
    // operand re-read its last row (never stored).
    const bool wb = wave >= 4;
    const uint8_t* gbase = static_cast<const uint8_t*>(wb ? B.data : A.data);
    const int64_t gld = wb ? B.ld : A.ld;
    const int64_t grow0 = wb ? tile_n * kBN : tile_m * kBM;
    const int64_t glim = wb ? N : M;
    uint32_t goff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * ((4 * wave + i) & 15) + (lane >> 2);
        int64_t gr = grow0 + r;
        gr = gr < glim ? gr : glim - 1;
        goff[i] = (uint32_t)(gr * gld) + 16u * (uint32_t)((lane & 3) ^ mx_swz(r));
    }
    const int cdst = (wb ? kMxB : kMxA) + 1024 * ((4 * wave) & 15);
    const uint8_t* sbase = wb ? B.scales : A.scales;
    uint32_t soff;
    {
        int64_t gr = grow0 + 64 * (wave & 3) + lane;
        gr = gr < glim ? gr : glim - 1;
        soff = (uint32_t)(gr * (wb ? B.ld_scales : A.ld_scales));
    }
    const int sdst = kMxS + (wb ? 1024 : 0) + 256 * (wave & 3);

    auto issue_codes = [&](int64_t k0, uint8_t* st) {
        const uint8_t* gb = gbase + (k0 >> 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((glb_void_t*)(gb + goff[i]),
                                             (lds_void_t*)(st + cdst + 1024 * i), 16, 0, 0);
    };
    auto issue_scales1 = [&](int64_t k0, uint8_t* st) {
        __builtin_amdgcn_global_load_lds((glb_void_t*)(sbase + (k0 >> 5) + soff),
                                         (lds_void_t*)(st + sdst), 4, 0, 0);
    };
    auto issue = [&](int64_t k0, uint8_t* st) {
        issue_codes(k0, st);
        issue_scales1(k0, st);
    };
    // the scales of steps k0 / 128 .. +2 of this wave's 64 rows
    const int gdst = (wb ? 4096 : 0) + 1024 * (wave & 3);
    auto issue_scales3 = [&](int64_t k0, uint8_t* sg) {
        __builtin_amdgcn_global_load_lds((glb_void_t*)(sbase + (k0 >> 5) + soff),
                                         (lds_void_t*)(sg + gdst), 12, 0, 0);
    };

    float16_t acc[4][2];
    zero_acc(acc);
    const int wm = wave >> 2, wn = wave & 3;
    const int a_row = wm * 128 + lr;  // + 32 tm
    const int b_row = wn * 64 + lr;   // + 32 tn
    const int sw = mx_swz(lr);        // = swz of every fragment row of this lane
    int aoff[2], boff[2];             // lane half g of sub-step s reads block 2s + g
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        aoff[sub] = kMxA + a_row * 64 + 16 * ((2 * sub + g) ^ sw);
        boff[sub] = kMxB + b_row * 64 + 16 * ((2 * sub + g) ^ sw);
    }

    // scale words: row r's at sc + pos(r) (A), sc + bofs + pos(r) (B); per-step
    // stage areas: pos(r) = 4 r; groups: 16 bytes a row
    auto compute_s = [&](const uint8_t* st, const uint8_t* sc, bool grp) {
        auto pos = [&](int r) { return grp ? 16 * r : 4 * r; };
        const uint8_t* Sa8 = sc;
        const uint8_t* Sb8 = sc + (grp ? 4096 : 1024);
        v8i_t af[2][4], bf[2][2];
        uint32_t sa[4], sb[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) af[sub][tm] = mx_frag(st + aoff[sub] + tm * 2048);
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) bf[sub][tn] = mx_frag(st + boff[sub] + tn * 2048);
        }
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) sa[tm] = *reinterpret_cast<const uint32_t*>(Sa8 + pos(a_row + 32 * tm));
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) sb[tn] = *reinterpret_cast<const uint32_t*>(Sb8 + pos(b_row + 32 * tn));
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int blk = 2 * sub + g;
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[sub][tm], bf[sub][tn], acc[tm][tn], 4, 4, 0,
                        (int)((sa[tm] >> (8 * blk)) & 0xFFu), 0, (int)((sb[tn] >> (8 * blk)) & 0xFFu));
        }
    };
    auto compute = [&](const uint8_t* st) { compute_s(st, st + kMxS, false); };

    // Partial last step, through registers: blocks past K get zero codes
    // (they add zero whatever their scale).  Thread t writes half t % 2 of
    // tile row t / 2 of both operands.
    auto tail = [&](int64_t k0, uint8_t* st) {
        const int row = tid >> 1, h = tid & 1;
        const int rs = mx_swz(row);
#pragma unroll
        for (int op = 0; op < 2; ++op) {
            int64_t gr = (op ? tile_n * kBN : tile_m * kBM) + row;
            const int64_t lim = op ? N : M;
            gr = gr < lim ? gr : lim - 1;
            const uint8_t* p = static_cast<const uint8_t*>(op ? B.data : A.data) +
                               gr * (op ? B.ld : A.ld) + (k0 >> 1);
            const uint8_t* ps = (op ? B.scales : A.scales) + gr * (op ? B.ld_scales : A.ld_scales);
            uint32_t sc = 0u;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int blk = 2 * h + j;  // block of the step = logical chunk of the row
                u32x4_t q = {0u, 0u, 0u, 0u};
                if ((k0 >> 5) + blk < nblk) {
                    q = *reinterpret_cast<const u32x4_t*>(p + 16 * blk);
                    sc |= (uint32_t)ps[(k0 >> 5) + blk] << (8 * j);
                }
                *reinterpret_cast<u32x4_t*>(st + (op ? kMxB : kMxA) + row * 64 + 16 * (blk ^ rs)) = q;
            }
            reinterpret_cast<uint16_t*>(st + kMxS + (op ? 1024 : 0))[row * 2 + h] = (uint16_t)sc;
        }
    };

    // Step t uses stage t % 3: wait until this wave's loads of step t have
    // landed (those of step t + 1, 5 per wave, may be in flight), barrier
    // (every wave's loads landed, every wave done with step t - 1), start
    // the loads of step t + 2 into the stage of step t - 1, compute step t.
    const int64_t nfull = K / kMxKS;
    if (nfull > 0) issue(0, lds0);
    if (nfull > 1) issue(kMxKS, lds1);
    auto sync = [&]() {
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    };
    int64_t t = 0;
    // While nine more whole steps follow, the scales come three steps per
    // load into sg0 / sg1 (steps 6i .. 6i+2 in sg0, 6i+3 .. 6i+5 in sg1): a
    // 4-byte scale load per row and step touched as many cache lines as all
    // the code loads of the step.  A wave's loads per step: 4 code pieces,
    // plus one scale piece at the first step of each three.
    if (nfull >= 9) {
        issue_scales3(0, sg0);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the prologue's loads
        for (; t + 9 <= nfull; t += 6) {  // scales read up to step t + 8
            __builtin_amdgcn_s_waitcnt(0x0f74);  // vmcnt(4)
            sync();
            issue_codes((t + 2) * kMxKS, lds2);
            issue_scales3((t + 3) * kMxKS, sg1);
            compute_s(lds0, sg0, true);
            __builtin_amdgcn_s_waitcnt(0x0f75);  // vmcnt(5)
            sync();
            issue_codes((t + 3) * kMxKS, lds0);
            compute_s(lds1, sg0 + 4, true);
            __builtin_amdgcn_s_waitcnt(0x0f74);
            sync();
            issue_codes((t + 4) * kMxKS, lds1);
            compute_s(lds2, sg0 + 8, true);
            __builtin_amdgcn_s_waitcnt(0x0f74);
            sync();
            issue_codes((t + 5) * kMxKS, lds2);
            issue_scales3((t + 6) * kMxKS, sg0);
            compute_s(lds0, sg1, true);
            __builtin_amdgcn_s_waitcnt(0x0f75);
            sync();
            issue_codes((t + 6) * kMxKS, lds0);
            compute_s(lds1, sg1 + 4, true);
            __builtin_amdgcn_s_waitcnt(0x0f74);
            sync();
            issue_codes((t + 7) * kMxKS, lds1);
            compute_s(lds2, sg1 + 8, true);
        }
        // steps t, t + 1 (codes in flight) get their scales in their stages
        __builtin_amdgcn_s_waitcnt(0x0f70);
        sync();
        issue_scales1(t * kMxKS, lds0);
        issue_scales1((t + 1) * kMxKS, lds1);
        __builtin_amdgcn_s_waitcnt(0x0f70);
    }
    for (; t + 4 < nfull; t += 3) {
        __builtin_amdgcn_s_waitcnt(0x0f75);  // vmcnt(5)
        sync();
        issue((t + 2) * kMxKS, lds2);
        compute(lds0);
        __builtin_amdgcn_s_waitcnt(0x0f75);
        sync();
        issue((t + 3) * kMxKS, lds0);
        compute(lds1);
        __builtin_amdgcn_s_waitcnt(0x0f75);
        sync();
        issue((t + 4) * kMxKS, lds1);
        compute(lds2);
    }
    for (; t < nfull; ++t) {  // the last (up to 4) full steps
        const int st = (int)(t % 3);
        uint8_t* cur = st == 0 ? lds0 : (st == 1 ? lds1 : lds2);
        uint8_t* ahead = st == 0 ? lds2 : (st == 1 ? lds0 : lds1);
        if (t + 1 < nfull)
            __builtin_amdgcn_s_waitcnt(0x0f75);
        else
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        __syncthreads();
        if (t + 2 < nfull) issue((t + 2) * kMxKS, ahead);
        compute(cur);
    }
    if (nfull * kMxKS < K) {
        const int st = (int)(nfull % 3);
        uint8_t* cur = st == 0 ? lds0 : (st == 1 ? lds1 : lds2);
        __syncthreads();  // (no loads in flight here) the stage is free
        tail(nfull * kMxKS, cur);
        __syncthreads();
        compute(cur);
    }

    __syncthreads();  // every wave is done reading the operand stages
    // waves 0-3 stage their output rows in lds0, waves 4-7 in lds1
    float* stage_out = reinterpret_cast<float*>(wave < 4 ? lds0 : lds1) + (wave & 3) * 32 * kEpiStride;
    store_tile<kOutF32>(acc, 1.0f, stage_out, tile_m * kBM + wm * 128, tile_n * kBN + wn * 64, M, N,
                        c, ldc);
}

namespace {

// ---------------------------------------------------------------------------
// bf16 operands
//
// Thread rid (0..255 of its operand) moves 8 pieces of 16 bytes (8 values)
// per step.  The two layouts keep different LDS tiles, each 36 KB a stage:
// Layout N (rows x K, K contiguous; Bf16RowsK): LDS rows of 64 k at a
//   144-byte pitch.  kg = rid % 8 names the 8-wide k group, c = rid / 8 the
//   rows: piece j is row c + 32 j, k group kg -- a wave's load covers 8 full
//   128-byte row segments, and the 8 lanes of equal c write 128 consecutive
//   LDS bytes.  A lane's MFMA fragment (row l % 32, k 8 (l / 32) .. +7) is
//   one 16-byte read.
// Layout T (K x rows, rows contiguous; Bf16KRows): the tile stays as it lies
//   in memory, 64 k-rows of 256 values at a 576-byte pitch.  ck = rid % 32
//   names the 8-row chunk and kr = rid / 32 the k-row: piece p is k-row
//   kr + 8 p -- 32 lanes read and write 512 contiguous bytes.  A fragment
//   comes from two transposing LDS reads (ds_read_b64_tr_b16): within each
//   16-lane group, result element j of lane i is element 16 j + i of the 16
//   lanes' 4-value pieces taken in lane order, so lane r of the group points
//   at k-row k0 + r / 4, rows m0 + 4 (r % 4) .. +3, and every lane receives
//   4 consecutive k of its own row.  Each transposing read touches 4 k-rows;
//   the pitch of 512 + 64 bytes starts them 64 bytes apart in the banks.
// K and the row count are multiples of 8, so a piece is wholly inside or
// wholly outside the operand.
// ---------------------------------------------------------------------------
struct Bf16Row {
    uint4 v[8];
};

// Per-thread load state of either layout: the first piece's address and two
// small indices whose meaning depends on the layout.
struct Bf16Load {
    const uint16_t* base;
    int64_t ld, K;
    int i0, i1;
};

struct Bf16RowsK {
    // rid: this thread's index within its operand, r0: the tile's first row,
    // lim: rows of the operand
    static __device__ __forceinline__ Bf16Load make(const OpArgs& o, int rid, int64_t r0, int64_t lim,
                                                    int64_t K)
    {
        const int kg = rid & 7, c = rid >> 3;
        const int64_t left = lim - r0 - 1;  // last valid row offset within the tile
        const int cmax = left < 255 ? (int)left : 255;
        return Bf16Load{static_cast<const uint16_t*>(o.data) + r0 * o.ld + 8 * kg, o.ld, K, c, cmax};
    }
    // piece j: row c + 32 j (rows past the operand re-read its last row)
    static __device__ __forceinline__ const uint4* piece(const Bf16Load& L, int64_t k0, int j)
    {
        return reinterpret_cast<const uint4*>(L.base + (int64_t)min(L.i0 + 32 * j, L.i1) * L.ld + k0);
    }
    static __device__ __forceinline__ void load_full(const Bf16Load& L, int64_t k0, Bf16Row& w)
    {
#pragma unroll
        for (int j = 0; j < 8; ++j) w.v[j] = *piece(L, k0, j);
    }
    // partial last step: pieces past K read as zero
    static __device__ __forceinline__ void load_tail(const Bf16Load& L, int kg, int64_t k0, Bf16Row& w)
    {
#pragma unroll
        for (int j = 0; j < 8; ++j) w.v[j] = (k0 + 8 * kg < L.K) ? *piece(L, k0, j) : make_uint4(0, 0, 0, 0);
    }
    static __device__ __forceinline__ void store(const Bf16Row& w, int rid, uint8_t* __restrict__ op)
    {
        const int kg = rid & 7, c = rid >> 3;
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(op + (c + 32 * j) * kRowBytes + 16 * kg) = w.v[j];
    }
    // A lane's fragment (row `row` + lane % 32, sub-step 0) sits at byte
    // frag_off(row, lane); 32 rows further on add kRows32, a sub-step kSub.
    static constexpr int kRows32 = 32 * kRowBytes, kSub = 32;
    static __device__ __forceinline__ int frag_off(int row, int lane)
    {
        return (row + (lane & 31)) * kRowBytes + 16 * (lane >> 5);
    }
    static __device__ __forceinline__ bf16x8_t frag(const uint8_t* at)
    {
        return *reinterpret_cast<const bf16x8_t*>(at);
    }
};

constexpr int kTPitch = 576;  // LDS bytes per k-row of a layout-T tile: 256 values + 64 pad
static_assert(64 * kTPitch == kOpBytes, "both layouts fill one operand stage");

typedef short short4_t __attribute__((ext_vector_type(4)));

struct Bf16KRows {
    static __device__ __forceinline__ Bf16Load make(const OpArgs& o, int rid, int64_t r0, int64_t lim,
                                                    int64_t K)
    {
        const int ck = rid & 31, kr = rid >> 5;
        int64_t m = r0 + 8 * ck;  // chunks past the operand re-read its last chunk
        m = m + 8 <= lim ? m : lim - 8;
        return Bf16Load{static_cast<const uint16_t*>(o.data) + (int64_t)kr * o.ld + m, o.ld, K, kr, 0};
    }
    static __device__ __forceinline__ const uint4* piece(const Bf16Load& L, int64_t k0, int p)
    {
        return reinterpret_cast<const uint4*>(L.base + (k0 + 8 * p) * L.ld);
    }
    static __device__ __forceinline__ void load_full(const Bf16Load& L, int64_t k0, Bf16Row& w)
    {
#pragma unroll
        for (int p = 0; p < 8; ++p) w.v[p] = *piece(L, k0, p);
    }
    static __device__ __forceinline__ void load_tail(const Bf16Load& L, int, int64_t k0, Bf16Row& w)
    {
#pragma unroll
        for (int p = 0; p < 8; ++p)
            w.v[p] = (k0 + L.i0 + 8 * p < L.K) ? *piece(L, k0, p) : make_uint4(0, 0, 0, 0);
    }
    static __device__ __forceinline__ void store(const Bf16Row& w, int rid, uint8_t* __restrict__ op)
    {
        const int ck = rid & 31, kr = rid >> 5;
#pragma unroll
        for (int p = 0; p < 8; ++p) *reinterpret_cast<uint4*>(op + (kr + 8 * p) * kTPitch + 16 * ck) = w.v[p];
    }
    // lane r of 16-lane group G points at k-row 8 (G / 2) + r / 4 (+ 4 for
    // the second read), rows row + 16 (G % 2) + 4 (r % 4) .. +3
    static constexpr int kRows32 = 64, kSub = 16 * kTPitch;
    static __device__ __forceinline__ int frag_off(int row, int lane)
    {
        const int G = lane >> 4, r = lane & 15;
        return (8 * (G >> 1) + (r >> 2)) * kTPitch + 2 * (row + 16 * (G & 1) + 4 * (r & 3));
    }
    static __device__ __forceinline__ bf16x8_t frag(const uint8_t* at)
    {
        typedef __attribute__((address_space(3))) short4_t lds_short4;
        lds_short4* p0 = (lds_short4*)(__attribute__((address_space(3))) uint8_t*)(at);
        lds_short4* p1 = (lds_short4*)(__attribute__((address_space(3))) uint8_t*)(at + 4 * kTPitch);
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
        typedef short short8_t __attribute__((ext_vector_type(8)));
        return __builtin_bit_cast(bf16x8_t, (short8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// Instruction-schedule hint for one bf16 K step (32 MFMAs per wave): the
// first half of the MFMAs is interleaved with the LDS fragment reads only;
// the second half also carries the next step's LDS writes and the transposes
// feeding them.
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

}  // namespace

template <class SA, class SB, bool kOutF32>
__global__ __launch_bounds__(512, 1) void k_gemm_bf16(OpArgs A, OpArgs B, int64_t M, int64_t N,
                                                      int64_t K, void* __restrict__ c, int64_t ldc)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kOpBytes];  // [stage][A/B]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int64_t tile_m, tile_n;
    tile_of(M, N, tile_m, tile_n);

    // threads 0..255 (waves 0-3) bring the A tile into LDS, 256..511 the B tile
    const bool is_b = tid >= 256;
    const int rid = tid & 255;
    constexpr bool kSame = std::is_same<SA, SB>::value;
    const OpArgs& op = is_b ? B : A;
    const int64_t r0 = is_b ? tile_n * kBN : tile_m * kBM, lim = is_b ? N : M;
    const Bf16Load src = (kSame || !is_b) ? SA::make(op, rid, r0, lim, K) : SB::make(op, rid, r0, lim, K);
    auto load_full = [&](int64_t k0, Bf16Row& w) {
        if (!kSame && is_b) SB::load_full(src, k0, w);
        else SA::load_full(src, k0, w);
    };
    auto load_tail = [&](int64_t k0, Bf16Row& w) {
        if (!kSame && is_b) SB::load_tail(src, rid & 7, k0, w);
        else SA::load_tail(src, rid & 7, k0, w);
    };
    auto put = [&](const Bf16Row& w, int stage) {
        if (!kSame && is_b) SB::store(w, rid, lds[stage][1]);
        else SA::store(w, rid, lds[stage][is_b ? 1 : 0]);
    };

    float16_t acc[4][2];
    zero_acc(acc);
    const int wm = wave >> 2, wn = wave & 3;  // the wave's 128-row A slab and 64-row B slab
    const int a_off = SA::frag_off(wm * 128, lane), b_off = SB::frag_off(wn * 64, lane);

    auto compute = [&](int stage) {
        const uint8_t* As = lds[stage][0] + a_off;
        const uint8_t* Bs = lds[stage][1] + b_off;
        bf16x8_t af[2][4], bf[2][2];  // fragments of two sub-steps in flight
#pragma unroll
        for (int t = 0; t < 4; ++t) af[0][t] = SA::frag(As + t * SA::kRows32);
#pragma unroll
        for (int t = 0; t < 2; ++t) bf[0][t] = SB::frag(Bs + t * SB::kRows32);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cur = i & 1, nxt = cur ^ 1;
            if (i < 3) {
#pragma unroll
                for (int t = 0; t < 4; ++t) af[nxt][t] = SA::frag(As + t * SA::kRows32 + (i + 1) * SA::kSub);
#pragma unroll
                for (int t = 0; t < 2; ++t) bf[nxt][t] = SB::frag(Bs + t * SB::kRows32 + (i + 1) * SB::kSub);
            }
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][tm], bf[cur][tn], acc[tm][tn], 0, 0, 0);
        }
    };
    // the interleaving hint counts one 16-byte LDS read per fragment
    constexpr bool kHints = std::is_same<SA, Bf16RowsK>::value && std::is_same<SB, Bf16RowsK>::value;

    // One register stage: the loads of step s+1 are issued before the MFMAs
    // of step s (a scheduling barrier keeps them there) and written to LDS
    // after them.
    const int64_t nsteps = (K + kKS - 1) / kKS;
    const int64_t nfull = K / kKS;
    int64_t s = 0;
    Bf16Row g0;
    if (nfull > 0) {
        load_full(0, g0);
        put(g0, 0);
    }
    __syncthreads();
    for (; s + 2 <= nfull; s += 2) {
        load_full((s + 1) * kKS, g0);
        __builtin_amdgcn_sched_barrier(0);
        compute(0);
        put(g0, 1);
        if constexpr (kHints) interleave_step(std::make_integer_sequence<int, 32>{});
        __syncthreads();
        load_full((s + 2 < nfull ? s + 2 : nfull - 1) * kKS, g0);
        __builtin_amdgcn_sched_barrier(0);
        compute(1);
        put(g0, 0);  // harmless on the last pass: stage 0 is not read again
        if constexpr (kHints) interleave_step(std::make_integer_sequence<int, 32>{});
        __syncthreads();
    }
    if (s < nfull) compute(0);  // odd number of full steps: the last one is in stage 0
    if (nfull < nsteps) {       // partial last step
        load_tail(nfull * kKS, g0);
        __syncthreads();
        put(g0, 1);
        __syncthreads();
        compute(1);
    }

    __syncthreads();  // every wave is done reading the operand stages
    store_tile<kOutF32>(acc, 1.0f, reinterpret_cast<float*>(&lds[0][0][0]) + wave * 32 * kEpiStride,
                        tile_m * kBM + wm * 128, tile_n * kBN + wn * 64,
                        M, N, c, ldc);
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

static void launch_fill_zero(int64_t M, int64_t N, void* c, int64_t ldc, bool out_fp32,
                             hipStream_t s)
{
    const dim3 g((unsigned)((M * N + 255) / 256));
    if (out_fp32)
        hipLaunchKernelGGL(k_fill_zero<true>, g, dim3(256), 0, s, c, ldc, M, N);
    else
        hipLaunchKernelGGL(k_fill_zero<false>, g, dim3(256), 0, s, c, ldc, M, N);
}

static dim3 tile_grid(int64_t M, int64_t N, int64_t tm = kBM)
{
    return dim3((unsigned)(((M + tm - 1) / tm) * ((N + kBN - 1) / kBN)));
}

// Tile height of the NVFP4 GEMM launches: 256 rows, one workgroup per CU
// (128-row tiles, two workgroups per CU, measured slower).
constexpr int kNvTM = kBM;

void launch_gemm_nt(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N, int64_t K,
                    void* c, int64_t ldc, bool out_fp32, hipStream_t s)
{
    if (M == 0 || N == 0) return;
    if (K == 0) return launch_fill_zero(M, N, c, ldc, out_fp32, s);
    const OpArgs A = nv_args(a), B = nv_args(b);
    const dim3 grid = tile_grid(M, N, kNvTM), block(2 * kNvTM);
    if (out_fp32)
        hipLaunchKernelGGL((k_gemm_nv<kNvTM, true>), grid, block, 0, s, A, B, M, N, K, c, ldc);
    else
        hipLaunchKernelGGL((k_gemm_nv<kNvTM, false>), grid, block, 0, s, A, B, M, N, K, c, ldc);
}

// The split tiles of a k_gemm_nv launch: output = (sum of the tile's parts,
// added in part order) * the output scale.  Each workgroup takes 4 rows of
// one tile (64 workgroups per tile, so that even a few split tiles spread
// over every CU; 16 rows per workgroup ran the 12B-layer reduces about 20 us
// slower); a thread adds one group of 4 consecutive values, all parts' loads
// in flight together.  The part count is a template parameter: with it a
// runtime bound, the conditional loads of an 8-entry array compiled into
// hundreds of register copies (196 VGPRs, two waves per SIMD) and the
// reduces ran at about 2 TB/s.
constexpr int kRedRows = 4;
template <bool kOutF32, int kSplit>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ ws, int64_t full_tiles,
                                                       const float* __restrict__ s_enc_a,
                                                       const float* __restrict__ s_enc_b, int64_t M,
                                                       int64_t N, void* __restrict__ c, int64_t ldc)
{
    constexpr int split = kSplit;
    constexpr int kGroups = kBN / 4;  // float4 groups per tile row
    const int64_t t = blockIdx.x / (kBM / kRedRows);
    const int rg = (int)(blockIdx.x % (kBM / kRedRows));
    int64_t tile_m, tile_n;
    tile_of<kBM>(M, N, tile_m, tile_n, full_tiles + t);
    float alpha;
    int alpha_exp;
    output_scale(*s_enc_a, *s_enc_b, alpha, alpha_exp);
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(ws + t * split * (int64_t)(kBM * kBN));
    constexpr int64_t kPart = kBM * kBN / 4;  // float4 per part
#pragma unroll
    for (int it = 0; it < kRedRows * kGroups / 256; ++it) {
        const int i = rg * kRedRows * kGroups + it * 256 + threadIdx.x;
        const int r = i / kGroups, q = i % kGroups;
        const int64_t row = tile_m * kBM + r, col = tile_n * kBN + 4 * q;
        f32x4_t part[kSplit];
#pragma unroll
        for (int p = 0; p < kSplit; ++p) part[p] = src[p * kPart + i];
        f32x4_t v = part[0];
#pragma unroll
        for (int p = 1; p < kSplit; ++p) v += part[p];
        if (row >= M || col >= N) continue;
        float y[4] = {v.x * alpha, v.y * alpha, v.z * alpha, v.w * alpha};
        if (alpha_exp != 0)
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = __builtin_ldexpf(y[j], alpha_exp);
        if constexpr (kOutF32) {
            float* dst = static_cast<float*>(c) + row * ldc + col;
            if (col + 4 <= N) {
                __builtin_nontemporal_store(f32x4_t{y[0], y[1], y[2], y[3]}, reinterpret_cast<f32x4_t*>(dst));
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (col + j < N) dst[j] = y[j];
            }
        } else {
            uint16_t* dst = static_cast<uint16_t*>(c) + row * ldc + col;
            const uint32_t w01 = bf16x2_rne(y[0], y[1]), w23 = bf16x2_rne(y[2], y[3]);
            const uint16_t b[4] = {(uint16_t)w01, (uint16_t)(w01 >> 16), (uint16_t)w23, (uint16_t)(w23 >> 16)};
            if (col + 4 <= N) {
                typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                __builtin_nontemporal_store(u32x2_t{b[0] | ((uint32_t)b[1] << 16), b[2] | ((uint32_t)b[3] << 16)},
                                            reinterpret_cast<u32x2_t*>(dst));
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (col + j < N) dst[j] = b[j];
            }
        }
    }
}

// Launches the reduce for `split` parts (splitk_plan keeps it in 2 .. 8).
template <bool kOutF32, int kS = 2>
void launch_splitk_reduce(int split, dim3 grid, hipStream_t s, const float* ws, int64_t full_tiles,
                          const float* s_enc_a, const float* s_enc_b, int64_t M, int64_t N, void* c,
                          int64_t ldc)
{
    if constexpr (kS <= 8) {
        if (split == kS) {
            hipLaunchKernelGGL((k_splitk_reduce<kOutF32, kS>), grid, dim3(256), 0, s, ws, full_tiles,
                               s_enc_a, s_enc_b, M, N, c, ldc);
            return;
        }
        launch_splitk_reduce<kOutF32, kS + 1>(split, grid, s, ws, full_tiles, s_enc_a, s_enc_b, M, N, c,
                                              ldc);
    }
}

int64_t splitk_plan(int64_t M, int64_t N, int64_t K, int cus, int64_t& full_tiles, int& split)
{
    const int64_t T = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    const int64_t rem = cus > 0 ? T % cus : 0;
    const int64_t nst = (K + kKS - 1) / kKS;
    full_tiles = T;
    split = 1;
    if (rem == 0) return 0;
    int64_t s = cus / rem;
    if (s > 8) s = 8;
    while (s > 1 && nst / s < 4) --s;  // every part keeps at least 4 K steps
    if (s < 2) return 0;
    full_tiles = T - rem;
    split = (int)s;
    return rem * s * (int64_t)(kBM * kBN) * (int64_t)sizeof(float);
}

void launch_gemm_nt_split(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N,
                          int64_t K, void* c, int64_t ldc, bool out_fp32, float* ws,
                          int64_t full_tiles, int split, hipStream_t s)
{
    if (split < 2) return launch_gemm_nt(a, b, M, N, K, c, ldc, out_fp32, s);
    const OpArgs A = nv_args(a), B = nv_args(b);
    const int64_t T = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    const int64_t rem = T - full_tiles;
    const dim3 grid((unsigned)(full_tiles + rem * split)), block(512);
    if (out_fp32)
        hipLaunchKernelGGL((k_gemm_nv<kBM, true>), grid, block, 0, s, A, B, M, N, K, c, ldc, nullptr,
                           nullptr, 0u, full_tiles, split, ws);
    else
        hipLaunchKernelGGL((k_gemm_nv<kBM, false>), grid, block, 0, s, A, B, M, N, K, c, ldc, nullptr,
                           nullptr, 0u, full_tiles, split, ws);
    const dim3 rgrid((unsigned)(rem * (kBM / kRedRows)));
    if (out_fp32)
        launch_splitk_reduce<true>(split, rgrid, s, ws, full_tiles, a.s_enc, b.s_enc, M, N, c, ldc);
    else
        launch_splitk_reduce<false>(split, rgrid, s, ws, full_tiles, a.s_enc, b.s_enc, M, N, c, ldc);
}

// Zeroes the output maxima (a kernel, not a memset, so the sequence can be
// captured in a graph).
__global__ void k_zero_amax(uint32_t* a, uint32_t* b)
{
    *a = 0u;
    if (b) *b = 0u;
}

void launch_gemm_nt_amax(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N,
                         int64_t K, uint16_t* c, int64_t ldc, float* amax, float* amax_rht,
                         uint32_t mask, hipStream_t s)
{
    uint32_t* ab = reinterpret_cast<uint32_t*>(amax);
    uint32_t* rb = reinterpret_cast<uint32_t*>(amax_rht);
    hipLaunchKernelGGL(k_zero_amax, dim3(1), dim3(1), 0, s, ab, rb);
    if (M == 0 || N == 0) return;
    if (K == 0) return launch_fill_zero(M, N, c, ldc, false, s);  // maxima stay 0
    const OpArgs A = nv_args(a), B = nv_args(b);
    const dim3 grid = tile_grid(M, N, kNvTM), block(2 * kNvTM);
    if (rb)
        hipLaunchKernelGGL((k_gemm_nv<kNvTM, false, 2>), grid, block, 0, s, A, B, M, N, K,
                           static_cast<void*>(c), ldc, ab, rb, mask);
    else
        hipLaunchKernelGGL((k_gemm_nv<kNvTM, false, 1>), grid, block, 0, s, A, B, M, N, K,
                           static_cast<void*>(c), ldc, ab, rb, mask);
}

void launch_gemm_mx(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N, int64_t K,
                    void* c, int64_t ldc, bool out_fp32, hipStream_t s)
{
    if (M == 0 || N == 0) return;
    if (K == 0) return launch_fill_zero(M, N, c, ldc, out_fp32, s);
    const OpArgs A{a.codes, a.ld_codes, a.scales, a.ld_scales, 0, nullptr};
    const OpArgs B{b.codes, b.ld_codes, b.scales, b.ld_scales, 0, nullptr};
    if (out_fp32)
        hipLaunchKernelGGL(k_gemm_mx<true>, tile_grid(M, N), dim3(512), 0, s, A, B, M, N, K, c, ldc);
    else
        hipLaunchKernelGGL(k_gemm_mx<false>, tile_grid(M, N), dim3(512), 0, s, A, B, M, N, K, c, ldc);
}

template <class SA, class SB>
static void launch_bf16(const OpArgs& a, const OpArgs& b, int64_t M, int64_t N, int64_t K, void* c,
                        int64_t ldc, bool out_fp32, hipStream_t s)
{
    if (out_fp32)
        hipLaunchKernelGGL((k_gemm_bf16<SA, SB, true>), tile_grid(M, N), dim3(512), 0, s, a, b, M, N, K, c, ldc);
    else
        hipLaunchKernelGGL((k_gemm_bf16<SA, SB, false>), tile_grid(M, N), dim3(512), 0, s, a, b, M, N, K, c, ldc);
}

void launch_bf16_gemm(const uint16_t* a, int64_t lda, bool a_t, const uint16_t* b, int64_t ldb,
                      bool b_t, int64_t M, int64_t N, int64_t K, void* c, int64_t ldc,
                      bool out_fp32, hipStream_t s)
{
    if (M == 0 || N == 0) return;
    if (K == 0) return launch_fill_zero(M, N, c, ldc, out_fp32, s);
    const OpArgs A{a, lda, nullptr, 0, 0, nullptr};
    const OpArgs B{b, ldb, nullptr, 0, 0, nullptr};
    if (!a_t && !b_t)
        launch_bf16<Bf16RowsK, Bf16RowsK>(A, B, M, N, K, c, ldc, out_fp32, s);
    else if (!a_t)
        launch_bf16<Bf16RowsK, Bf16KRows>(A, B, M, N, K, c, ldc, out_fp32, s);
    else if (b_t)
        launch_bf16<Bf16KRows, Bf16KRows>(A, B, M, N, K, c, ldc, out_fp32, s);
    else
        launch_bf16<Bf16KRows, Bf16RowsK>(A, B, M, N, K, c, ldc, out_fp32, s);
}

// ---------------------------------------------------------------------------
// Sustained matrix-core throughput (a measurement aid, not a pass): 8 waves
// per workgroup (two per SIMD) run rounds of 64 matrix instructions on a
// pool of 8 A and 8 B register fragments, a different pair for every
// instruction, into 8 accumulators each (every accumulator is reused 8
// instructions later, so no instruction waits on another).  kOps = 0: the
// GEMM's v_mfma_f32_32x32x16_f16 on exact fp16 values E2M1 x E4M3 / 64 with
// a random sign, as the decoded operands; 1: the same instruction on random
// fp16 in [-1, 1); 2: the block-scaled FP4 instruction of the MXFP4 GEMM,
// v_mfma_scale_f32_32x32x64_f8f6f4, on random E2M1 codes with unit scales.
// With every operand in registers the loop measures what the matrix cores
// sustain at the clock the chip holds under that load, which the power
// limit sets below the nominal 2.4 GHz.
// ---------------------------------------------------------------------------

namespace {
__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}
}  // namespace

template <int kOps>
__global__ __launch_bounds__(512, 1) void k_mfma_sustain(float* __restrict__ out, int64_t iters)
{
    float16_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    const uint32_t tid = (uint32_t)(blockIdx.x * blockDim.x + threadIdx.x);
    if constexpr (kOps == 2) {
        v8i_t fa[8], fb[8];  // 32 E2M1 codes (4 dwords) per lane; the upper half unused
#pragma unroll
        for (int p = 0; p < 8; ++p)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t h1 = mix32(tid * 131u + 17u * p + e), h2 = mix32(h1 + 0x9e3779b9u);
                fa[p][e] = e < 4 ? (int)h1 : 0;
                fb[p][e] = e < 4 ? (int)h2 : 0;
            }
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 64; ++j)
                acc[j & 7] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    fa[j & 7], fb[((j >> 3) + j) & 7], acc[j & 7], 4, 4, 0, 127, 0, 127);
        }
    } else {
        half8_t fa[8], fb[8];
        const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
#pragma unroll
        for (int p = 0; p < 8; ++p)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t h1 = mix32(tid * 131u + 17u * p + e), h2 = mix32(h1 + 0x9e3779b9u);
                float va, vb;
                if constexpr (kOps == 0) {
                    const float sa = (1.0f + (float)(h1 >> 29) * 0.125f) * (float)(1u << ((h1 >> 20) & 3u)) * 0.015625f;
                    const float sb = (1.0f + (float)(h2 >> 29) * 0.125f) * (float)(1u << ((h2 >> 20) & 3u)) * 0.015625f;
                    va = (h1 & 8u) ? -mag[h1 & 7u] * sa : mag[h1 & 7u] * sa;
                    vb = (h2 & 8u) ? -mag[h2 & 7u] * sb : mag[h2 & 7u] * sb;
                } else {
                    va = (float)(h1 & 0xFFFFu) * (1.0f / 32768.0f) - 1.0f;
                    vb = (float)(h2 & 0xFFFFu) * (1.0f / 32768.0f) - 1.0f;
                }
                fa[p][e] = (_Float16)va;
                fb[p][e] = (_Float16)vb;
            }
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int j = 0; j < 64; ++j)
                acc[j & 7] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[j & 7], fb[((j >> 3) + j) & 7], acc[j & 7], 0, 0, 0);
        }
    }
    float r = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) r += acc[j][e];
    out[tid] = r;
}

void launch_mfma_sustain(int64_t blocks, int64_t iters, int operands, float* out, hipStream_t s)
{
    const dim3 g((unsigned)blocks), b(512);
    if (operands == 0)
        hipLaunchKernelGGL(k_mfma_sustain<0>, g, b, 0, s, out, iters);
    else if (operands == 1)
        hipLaunchKernelGGL(k_mfma_sustain<1>, g, b, 0, s, out, iters);
    else
        hipLaunchKernelGGL(k_mfma_sustain<2>, g, b, 0, s, out, iters);
}

}  // namespace nvfp4
