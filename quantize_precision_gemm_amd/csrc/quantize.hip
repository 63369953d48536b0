// quantize.hip -- NVFP4 quantisers for gfx950: tensor amax, 1x16 and 16x16
// block quantisation (RNE or stochastic rounding), and the random-Hadamard
// transposing quantiser for weight-gradient operands.
//
// Recipe: "Pretraining Large Language Models with NVFP4" (gist.science
// summary), Technische Zusammenfassung 2.A (16-element blocks, E4M3 block
// scale, FP32 tensor scale), 2.B.2 (16x16 random Hadamard transform on the
// weight-gradient inputs), 2.B.3 (16x16 blocks for weights), 2.B.4 (stochastic
// rounding for gradients, RNE otherwise).
//
// Every quantiser is two streaming passes over the bf16 input: a tensor-amax
// reduction (one atomic max per workgroup on the fp32 bit pattern, which
// orders like the value for non-negative floats) and an encode pass that
// reads the amax back from device memory.  Both are HBM-bound streams.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// Streaming loads
//
// Every pass here streams its bf16 input once.  Loads with the non-temporal
// hint (the streaming cache policy) sustain a higher read rate: a 1 GiB
// max-reduction reads 6.95 TB/s with them against 6.2 TB/s without on
// MI355X.
// ---------------------------------------------------------------------------

typedef unsigned u32x4_nt_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream(const void* p)
{
    const u32x4_nt_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// amax
// ---------------------------------------------------------------------------

__global__ void k_zero_u32(uint32_t* p) { *p = 0u; }
__global__ void k_zero_u32x2(uint32_t* p, uint32_t* q)
{
    *p = 0u;
    *q = 0u;
}

// Empty tensors: only the tensor amax and encode scale are published.
__global__ void k_publish(const float* __restrict__ amax_src, float* __restrict__ amax_out,
                          float* __restrict__ s_enc_out)
{
    const float amax = *amax_src;
    *amax_out = amax;
    *s_enc_out = tensor_scale(amax);
}

// Merge a workgroup's max into the tensor amax.  Same-address atomics from
// thousands of workgroups serialise in L2, so the atomic is skipped when the
// value already stored is at least as large (a stale read only costs an
// unnecessary atomic; the final value is the same).
__device__ __forceinline__ void merge_amax(uint32_t* amax_bits, uint32_t v)
{
    if (v > __atomic_load_n(amax_bits, __ATOMIC_RELAXED)) atomicMax(amax_bits, v);
}

// max |x| of a row-major bf16 matrix (rows x cols, leading dimension ld, all
// multiples of 8 elements), as fp32 bits, atomically merged into *amax_bits.
__global__ __launch_bounds__(256) void k_amax_rows(const uint16_t* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t ld,
                                                   uint32_t* __restrict__ amax_bits)
{
    const int64_t vpr = cols >> 3;  // 16-byte vectors per row
    const int64_t nvec = rows * vpr;
    uint32_t m = 0u;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < nvec; v += stride) {
        int64_t r = v / vpr;
        int64_t cv = v - r * vpr;
        uint4 q = ld_stream(x + r * ld + cv * 8);
        m = max(m, max(max(bf16_absmax2(q.x), bf16_absmax2(q.y)),
                       max(bf16_absmax2(q.z), bf16_absmax2(q.w))));
    }
    m = wave_max_u32(m);
    __shared__ uint32_t red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t mm = max(max(red[0], red[1]), max(red[2], red[3]));
        merge_amax(amax_bits, mm << 16);
    }
}

// Contiguous fast path (ld == cols): a flat stream of 16-byte vectors, four
// in flight per thread.
__device__ __forceinline__ uint32_t absmax8(const uint4& q)
{
    return max(max(bf16_absmax2(q.x), bf16_absmax2(q.y)), max(bf16_absmax2(q.z), bf16_absmax2(q.w)));
}

// Streaming reads run best with a few resident workgroups per CU that each
// walk the tensor (grid-stride) with several loads in flight, rather than
// one short-lived workgroup per chunk.
constexpr int kFlatLoads = 4;      // 16-byte loads in flight per thread
constexpr int kFlatGrid = 1024;    // workgroups of the flat amax pass
constexpr int kAmaxGrid = 512;     // workgroups of the RHT amax passes
__global__ __launch_bounds__(256) void k_amax_flat(const uint4* __restrict__ x, int64_t nvec,
                                                   uint32_t* __restrict__ amax_bits)
{
    constexpr int kL = kFlatLoads;
    uint32_t m = 0u;
    const int64_t stride = (int64_t)gridDim.x * 256 * kL;
    int64_t base = (int64_t)blockIdx.x * 256 * kL + threadIdx.x;
    for (; base + 256 * (kL - 1) < nvec; base += stride) {
        uint4 q[kL];
#pragma unroll
        for (int j = 0; j < kL; ++j) q[j] = ld_stream(x + base + 256 * j);
#pragma unroll
        for (int j = 0; j < kL; ++j) m = max(m, absmax8(q[j]));
    }
    if (base < nvec) {
#pragma unroll
        for (int j = 0; j < kL; ++j)
            if (base + 256 * j < nvec) m = max(m, absmax8(x[base + 256 * j]));
    }
    m = wave_max_u32(m);
    __shared__ uint32_t red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t mm = max(max(red[0], red[1]), max(red[2], red[3]));
        merge_amax(amax_bits, mm << 16);
    }
}

// ---------------------------------------------------------------------------
// Encode helpers
// ---------------------------------------------------------------------------

// 16 bf16 values (two 16-byte vectors) -> fp32
__device__ __forceinline__ void unpack16(const uint4& a, const uint4& b, float (&v)[16])
{
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
}

__device__ __forceinline__ float absmax16(const float (&v)[16])
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(v[i]));
    return m;
}

// 16 values times f, RNE-encoded into 8 packed bytes.
__device__ __forceinline__ uint2 encode16_rne(const float (&v)[16], float f)
{
    uint32_t lo = 0u, hi = 0u;
    lo = e2m1_rne_pk<0>(lo, v[0] * f, v[1] * f);
    lo = e2m1_rne_pk<1>(lo, v[2] * f, v[3] * f);
    lo = e2m1_rne_pk<2>(lo, v[4] * f, v[5] * f);
    lo = e2m1_rne_pk<3>(lo, v[6] * f, v[7] * f);
    hi = e2m1_rne_pk<0>(hi, v[8] * f, v[9] * f);
    hi = e2m1_rne_pk<1>(hi, v[10] * f, v[11] * f);
    hi = e2m1_rne_pk<2>(hi, v[12] * f, v[13] * f);
    hi = e2m1_rne_pk<3>(hi, v[14] * f, v[15] * f);
    return make_uint2(lo, hi);
}

// 16 values times f, stochastically rounded with the draws of elements
// 8*g8 .. 8*g8+15 (two Philox blocks), into 8 packed bytes.
__device__ __forceinline__ uint2 encode16_sr(const float (&v)[16], float f, uint64_t seed,
                                             uint64_t g8)
{
    const Draws8 d0 = sr_draws8(seed, g8);
    const Draws8 d1 = sr_draws8(seed, g8 + 1);
    float y0[8], y1[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        y0[i] = v[i] * f;
        y1[i] = v[8 + i] * f;
    }
    return make_uint2(e2m1_sr8(y0, d0.w), e2m1_sr8(y1, d1.w));
}

// ---------------------------------------------------------------------------
// 1x16 quantiser: one thread per 16-element block.  A workgroup of 4 waves
// covers 4 rows x 64 blocks, one row per wave, so each wave reads 2 KB of a
// row.  Interleaved codes go through LDS, and each wave then writes 4 whole
// 128-byte lines (one K step of the 4 rows in each).  Measured on the
// 12B-layer dY (RNE, cold): 83 us; a wave per 4 rows x 16 blocks writing
// whole lines straight from registers took 87 us (4 rows x 512-byte reads
// per wave); the row-major form's mapping (a wave per 64 blocks of one row,
// rows of a line group in workgroups far apart, often on other XCDs whose
// L2s each wrote back a part of the line) took 108 us.  Row-major codes are
// written straight from registers (a wave writes 512 bytes of its row).
// ---------------------------------------------------------------------------

template <bool kSR, bool kRht = false>
__global__ __launch_bounds__(256) void k_quant_1x16(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax_src, uint64_t seed, uint8_t* __restrict__ codes,
    int64_t ld_codes, bool il, uint8_t* __restrict__ scales, int64_t ld_scales,
    float* __restrict__ amax_out, float* __restrict__ s_enc_out, uint32_t mask = 0u)
{
    __shared__ uint2 sc[4][64];  // interleaved codes of the workgroup's 4 rows
    const int64_t nb = cols >> 4;
    const int64_t nchunk = (nb + 63) >> 6;  // 64-block chunks per row
    const float amax = *amax_src;
    const float s_enc = tensor_scale(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *amax_out = amax;
        *s_enc_out = s_enc;
    }
    const int64_t g = blockIdx.x / nchunk, c = blockIdx.x - g * nchunk;
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int64_t r = 4 * g + w;
    const int64_t b = 64 * c + l;
    if (r < rows && b < nb) {
        const uint4* src = reinterpret_cast<const uint4*>(x + r * ld + b * 16);
        float v[16];
        unpack16(ld_stream(src), ld_stream(src + 1), v);
        if constexpr (kRht) rht16(v, mask);
        const uint32_t sb = block_scale(absmax16(v), s_enc);
        const float f = block_factor(sb, s_enc);
        uint2 pk;
        if constexpr (kSR)
            pk = encode16_sr(v, f, seed, (uint64_t)(r * cols + b * 16) >> 3);
        else
            pk = encode16_rne(v, f);
        scales[r * ld_scales + b] = (uint8_t)sb;
        if (!il) *reinterpret_cast<uint2*>(codes + r * ld_codes + b * 8) = pk;
        else sc[w][l] = pk;
    }
    if (!il) return;  // uniform over the launch
    __syncthreads();
    // thread t: line t / 16 of the chunk, row (t / 4) % 4, block 4 (t / 16) + t % 4
    const int t = threadIdx.x;
    const int orow = (t >> 2) & 3, oblk = 4 * (t >> 4) + (t & 3);
    const int64_t ro = 4 * g + orow, bo = 64 * c + oblk;
    if (ro < rows && bo < nb)
        *reinterpret_cast<uint2*>(codes + code_offset(ro, bo * 8, ld_codes, true)) = sc[orow][oblk];
}

// ---------------------------------------------------------------------------
// 16x16 quantiser (weights).  A workgroup of 512 threads covers 128 rows x
// 256 columns (8 x 16 tiles).  Thread t takes tile column t % 16 and rows
// 4*(t/16) .. +3, so the 4 threads sharing one tile sit in lanes 16 apart
// of the same wave and the tile amax is two lane shuffles; a row's codes
// leave as 128 contiguous bytes.  The transposed copy and its scales are
// assembled in LDS and written as 64-byte code rows and 8-byte scale rows.
// (128 x 128 tiles of 256 threads, with the transposed scales written byte
// by byte, ran 4 % slower on the 12B-layer weight.)  Interleaved outputs
// without a transform go to k_quant_16x16_il below.
// ---------------------------------------------------------------------------

constexpr int kW2TC = 16, kW2RG = 32;  // tile columns x row groups of 4 per workgroup
constexpr int kW2Rows = 4 * kW2RG, kW2Cols = 16 * kW2TC;

template <bool kSR, bool kRht = false>
__global__ __launch_bounds__(kW2TC * kW2RG) void k_quant_16x16(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax_src, uint64_t seed, uint8_t* __restrict__ codes,
    int64_t ld_codes, bool il, uint8_t* __restrict__ scales, int64_t ld_scales,
    uint8_t* __restrict__ codes_t, int64_t ld_codes_t, uint8_t* __restrict__ scales_t,
    int64_t ld_scales_t, float* __restrict__ amax_out, float* __restrict__ s_enc_out,
    uint32_t mask = 0u)
{
    constexpr int kTR = kW2RG / 4;  // tile rows per workgroup
    __shared__ __attribute__((aligned(16))) uint8_t tcodes[kW2Cols][kW2Rows / 2 + 16];  // [col][row/2]
    __shared__ uint8_t tsc[kW2TC][kTR];

    const int t = threadIdx.x;
    const int tcl = t % kW2TC, rg = t / kW2TC;
    const int64_t col0 = (int64_t)blockIdx.x * kW2Cols + tcl * 16;
    const int64_t row0 = (int64_t)blockIdx.y * kW2Rows + rg * 4;
    const bool valid = col0 < cols && row0 < rows;
    const float amax = *amax_src;
    const float s_enc = tensor_scale(amax);
    if (blockIdx.x == 0 && blockIdx.y == 0 && t == 0) {
        *amax_out = amax;
        *s_enc_out = s_enc;
    }

    float v[4][16];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (valid) {
            const uint4* src = reinterpret_cast<const uint4*>(x + (row0 + i) * ld + col0);
            unpack16(ld_stream(src), ld_stream(src + 1), v[i]);
            if constexpr (kRht) rht16(v[i], mask);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[i][j] = 0.0f;
        }
        m = __builtin_fmaxf(m, absmax16(v[i]));
    }
    uint32_t mb = __float_as_uint(m);
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, kW2TC, 64));
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, 2 * kW2TC, 64));
    const uint32_t sb = block_scale(__uint_as_float(mb), s_enc);
    const float f = block_factor(sb, s_enc);

    uint2 pk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (kSR)
            pk[i] = encode16_sr(v[i], f, seed, (uint64_t)((row0 + i) * cols + col0) >> 3);
        else
            pk[i] = encode16_rne(v[i], f);
        if (valid) *reinterpret_cast<uint2*>(codes + code_offset(row0 + i, col0 >> 1, ld_codes, il)) = pk[i];
    }
    const int64_t tr = row0 >> 4, tc = col0 >> 4;
    if (valid && (rg & 3) == 0) {
        scales[tr * ld_scales + tc] = (uint8_t)sb;
        tsc[tcl][rg >> 2] = (uint8_t)sb;
        if (scales_t && codes_t == nullptr) scales_t[tc * ld_scales_t + tr] = (uint8_t)sb;
    }
    if (codes_t == nullptr) return;

#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int sh = 4 * (k & 7);
        const uint32_t c0 = ((k < 8 ? pk[0].x : pk[0].y) >> sh) & 15u;
        const uint32_t c1 = ((k < 8 ? pk[1].x : pk[1].y) >> sh) & 15u;
        const uint32_t c2 = ((k < 8 ? pk[2].x : pk[2].y) >> sh) & 15u;
        const uint32_t c3 = ((k < 8 ? pk[3].x : pk[3].y) >> sh) & 15u;
        const uint16_t two = (uint16_t)(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
        *reinterpret_cast<uint16_t*>(&tcodes[tcl * 16 + k][rg * 2]) = two;
    }
    __syncthreads();
    if (scales_t && t < kW2TC * kTR) {  // one byte per thread, consecutive along a row of scales_t
        const int c = t / kTR, r = t % kTR;
        const int64_t tcg = (int64_t)blockIdx.x * kW2TC + c, trg = (int64_t)blockIdx.y * kTR + r;
        if (tcg * 16 < cols && trg * 16 < rows) scales_t[tcg * ld_scales_t + trg] = tsc[c][r];
    }
    constexpr int kPieces = kW2Rows / 32;  // 16-byte pieces per transposed row
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int idx = it * kW2TC * kW2RG + t;
        const int kr = idx / kPieces, q = idx % kPieces;
        const int64_t kcol = (int64_t)blockIdx.x * kW2Cols + kr;
        const int64_t nrow = (int64_t)blockIdx.y * kW2Rows + q * 32;
        if (kcol < cols && nrow < rows) {
            const uint4 val = *reinterpret_cast<const uint4*>(&tcodes[kr][q * 16]);
            uint8_t* dst = codes_t + code_offset(kcol, nrow >> 1, ld_codes_t, il);
            if (nrow + 32 <= rows) {
                *reinterpret_cast<uint4*>(dst) = val;
            } else {
                *reinterpret_cast<uint2*>(dst) = make_uint2(val.x, val.y);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 16x16 quantiser for interleaved codes (weights, no transform).  A wave
// covers one tile row (16 rows) by 512 columns: lane l holds 8 columns (16
// bytes) of each of the 16 rows, so every load instruction reads 1 KB of one
// row, and lanes 2k and 2k+1 hold the two halves of tile column k (its
// maximum is one lane-pair exchange).  A lane encodes one 32-bit word of 8
// codes per row, then transposes its 16 x 8 nibbles in registers into the 8
// columns' 8-byte pieces of the transposed copy.  The workgroup's 4 waves
// take 4 consecutive tile rows, so it holds whole 128-byte lines (4 rows of
// 64 elements) of both copies; they are assembled in LDS and leave as 16-byte
// stores, 8 whole lines per instruction.  Inputs are finite, so the integer
// maximum of the bf16 magnitudes is their float maximum.  Measured on the
// 12B-layer weight (20480 x 5120, cold, kernel alone): 66 us against 80 us
// for the row-major kernel above on the same layout; stored straight from
// registers (8-byte pieces, 64 lines per store instruction for the
// transposed copy) it took 86 us, with only the transposed copy staged 68 us.
// ---------------------------------------------------------------------------

constexpr int kW3Cols = 512, kW3Waves = 4;
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// In-place 8 x 8 transpose of 4-bit elements: element (i, j) is nibble j of
// w[i].  Swapping the off-diagonal 4 x 4, then 2 x 2, then 1 x 1 blocks.
__device__ __forceinline__ void transpose_nibbles8(uint32_t* w)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t t = ((w[i] >> 16) ^ w[i + 4]) & 0x0000FFFFu;
        w[i] ^= t << 16;
        w[i + 4] ^= t;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = (k & 1) + 4 * (k >> 1);
        const uint32_t t = ((w[i] >> 8) ^ w[i + 2]) & 0x00FF00FFu;
        w[i] ^= t << 8;
        w[i + 2] ^= t;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = 2 * k;
        const uint32_t t = ((w[i] >> 4) ^ w[i + 1]) & 0x0F0F0F0Fu;
        w[i] ^= t << 4;
        w[i + 1] ^= t;
    }
}

template <bool kSR>
__global__ __launch_bounds__(64 * kW3Waves) void k_quant_16x16_il(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const float* __restrict__ amax_src, uint64_t seed, uint8_t* __restrict__ codes,
    int64_t ld_codes, uint8_t* __restrict__ scales, int64_t ld_scales,
    uint8_t* __restrict__ codes_t, int64_t ld_codes_t, uint8_t* __restrict__ scales_t,
    int64_t ld_scales_t, float* __restrict__ amax_out, float* __restrict__ s_enc_out)
{
    const int64_t nbx = (cols + kW3Cols - 1) / kW3Cols;
    const int64_t bx = blockIdx.x % nbx, by = blockIdx.x / nbx;  // column chunks fastest
    const int l = threadIdx.x & 63;
    const int64_t tr = by * kW3Waves + (threadIdx.x >> 6);       // tile row
    const int64_t r0 = 16 * tr, c0 = bx * kW3Cols + 8 * l;
    const bool valid = r0 < rows && c0 < cols;  // lanes 2k, 2k+1 agree: cols % 16 == 0
    const float amax = *amax_src;
    const float s_enc = tensor_scale(amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *amax_out = amax;
        *s_enc_out = s_enc;
    }

    uint4 raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        raw[i] = valid ? ld_stream(x + (r0 + i) * ld + c0) : make_uint4(0u, 0u, 0u, 0u);
    u16x2_t m2 = {0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t u[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, u[k] & 0x7FFF7FFFu));
    }
    uint32_t mb = max((uint32_t)m2.x, (uint32_t)m2.y);
    mb = max(mb, (uint32_t)__shfl_xor((int)mb, 1, 64));
    const uint32_t sb = block_scale(__uint_as_float(mb << 16), s_enc);
    const float f = block_factor(sb, s_enc);

    uint32_t wd[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t u[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
        if constexpr (kSR) {
            float y[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                y[2 * k] = bf16_lo(u[k]) * f;
                y[2 * k + 1] = bf16_hi(u[k]) * f;
            }
            wd[i] = e2m1_sr8(y, sr_draws8(seed, (uint64_t)((r0 + i) * cols + c0) >> 3).w);
        } else {
            uint32_t c = 0u;
            c = e2m1_rne_pk<0>(c, bf16_lo(u[0]) * f, bf16_hi(u[0]) * f);
            c = e2m1_rne_pk<1>(c, bf16_lo(u[1]) * f, bf16_hi(u[1]) * f);
            c = e2m1_rne_pk<2>(c, bf16_lo(u[2]) * f, bf16_hi(u[2]) * f);
            c = e2m1_rne_pk<3>(c, bf16_lo(u[3]) * f, bf16_hi(u[3]) * f);
            wd[i] = c;
        }
    }
    if (valid && (l & 1) == 0) {
        const int64_t tc = c0 >> 4;
        scales[tr * ld_scales + tc] = (uint8_t)sb;
        if (scales_t) scales_t[tc * ld_scales_t + tr] = (uint8_t)sb;
    }
    // Both code copies are staged in LDS in line order (136-byte pitch
    // against bank conflicts) and stored 16 bytes a lane, 8 whole lines per
    // instruction.  The workgroup's codes are 128 lines (4 rows x 64
    // elements): 16 row groups x 8 line columns.
    constexpr int kPitch = 136;
    __shared__ __attribute__((aligned(16))) uint8_t cl[128 * kPitch];
    __shared__ __attribute__((aligned(16))) uint8_t tl[kW3Cols / 4 * kPitch];
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 16; ++i)  // local row 16w + i, bytes 4l .. 4l+3 of the chunk
        *reinterpret_cast<uint32_t*>(&cl[((4 * w + (i >> 2)) * 8 + (l >> 3)) * kPitch + (i & 3) * 32 + 4 * (l & 7)]) = wd[i];
    const bool with_t = codes_t != nullptr;  // uniform over the launch
    if (with_t) {
        transpose_nibbles8(wd);      // rows 0-7: wd[j] = column j's 8 codes
        transpose_nibbles8(wd + 8);  // rows 8-15
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kc = 8 * l + j;
            *reinterpret_cast<uint2*>(&tl[(kc >> 2) * kPitch + (kc & 3) * 32 + 8 * w]) = make_uint2(wd[j], wd[8 + j]);
        }
    }
    __syncthreads();
    const int64_t tr_end = rows >> 4;  // tile rows of the tensor
#pragma unroll
    for (int it = 0; it < 128 * 8 / (64 * kW3Waves); ++it) {
        const int id = it * 64 * kW3Waves + threadIdx.x;
        const int g = id >> 3, c = id & 7;         // line (row group g / 8, line column g % 8), chunk
        const int64_t rg = by * 4 * kW3Waves + (g >> 3);                // global row group
        const int64_t jb = bx * (kW3Cols / 64) + (g & 7);               // global line column
        const int64_t nbytes = (cols >> 1) - (jb * 32 + 16 * (c & 1));  // 0, 8, 16 or more valid
        if (4 * rg >= rows || nbytes <= 0) continue;
        uint8_t* dst = codes + rg * 4 * ld_codes + jb * 128 + 16 * c;
        const uint2 a = *reinterpret_cast<const uint2*>(&cl[g * kPitch + 16 * c]);
        if (nbytes >= 16) {
            const uint2 b = *reinterpret_cast<const uint2*>(&cl[g * kPitch + 16 * c + 8]);
            *reinterpret_cast<uint4*>(dst) = make_uint4(a.x, a.y, b.x, b.y);
        } else {
            *reinterpret_cast<uint2*>(dst) = a;
        }
    }
    if (!with_t) return;
#pragma unroll
    for (int it = 0; it < kW3Cols / 4 * 8 / (64 * kW3Waves); ++it) {
        const int id = it * 64 * kW3Waves + threadIdx.x;
        const int g = id >> 3, c = id & 7;           // line, 16-byte chunk: column 4g + c/2
        const int64_t kcol = bx * kW3Cols + 4 * g + (c >> 1);
        const int64_t t0 = by * kW3Waves + 2 * (c & 1);  // the chunk's first tile row
        if (kcol >= cols || t0 >= tr_end) continue;
        const uint2 a = *reinterpret_cast<const uint2*>(&tl[g * kPitch + 16 * c]);
        uint8_t* dst = codes_t + code_offset(kcol, 8 * t0, ld_codes_t, true);
        if (t0 + 1 < tr_end) {
            const uint2 b = *reinterpret_cast<const uint2*>(&tl[g * kPitch + 16 * c + 8]);
            *reinterpret_cast<uint4*>(dst) = make_uint4(a.x, a.y, b.x, b.y);
        } else {
            *reinterpret_cast<uint2*>(dst) = a;
        }
    }
}

// ---------------------------------------------------------------------------
// RHT + transpose + 1x16 quantiser (weight-gradient operands), and the amax
// passes over the transform.  A thread loads 8 channels (one 16-byte load per
// token row) of one 16-token chunk and runs their 8 butterflies.  The amax
// passes, which write nothing, give a workgroup 64 tokens x 512 channels so
// that every row is read in 1 KB runs, and walk the tiles grid-stride; the
// quantiser covers 256 tokens x 128 channels so that each channel's codes
// leave as 128 contiguous bytes.
// ---------------------------------------------------------------------------

constexpr int kRhtTok = 256, kRhtCh = 128;
constexpr int kAmTok = 64, kAmCh = 512;   // amax passes: 1 KB of every row per workgroup

__device__ __forceinline__ void load_rht_raw(const uint16_t* __restrict__ x, int64_t ld,
                                             int64_t tok0, int64_t ch0, uint4 (&raw)[16])
{
#pragma unroll
    for (int i = 0; i < 16; ++i) raw[i] = ld_stream(x + (tok0 + i) * ld + ch0);
}

// channel c (0..7) of the 8 loaded per row -> 16 fp32 values over the chunk
__device__ __forceinline__ void unpack_channel(const uint4 (&raw)[16], int c, float (&v)[16])
{
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t w = (c >> 1) == 0 ? raw[i].x : (c >> 1) == 1 ? raw[i].y : (c >> 1) == 2 ? raw[i].z : raw[i].w;
        v[i] = (c & 1) ? bf16_hi(w) : bf16_lo(w);
    }
}

__global__ __launch_bounds__(256) void k_rht_amax(const uint16_t* __restrict__ x, int64_t tokens,
                                                  int64_t channels, int64_t ld, uint32_t mask,
                                                  uint32_t* __restrict__ amax_bits)
{
    const int cg = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int64_t bch = (channels + kAmCh - 1) / kAmCh, btok = (tokens + kAmTok - 1) / kAmTok;
    uint32_t m = 0u;
    for (int64_t bt = blockIdx.x; bt < bch * btok; bt += gridDim.x) {
    const int64_t ch0 = (bt % bch) * kAmCh + cg * 8;
    const int64_t tok0 = (bt / bch) * kAmTok + j * 16;
    if (ch0 < channels && tok0 < tokens) {
        uint4 raw[16];
        load_rht_raw(x, ld, tok0, ch0, raw);
        float mu = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float v[16];
            unpack_channel(raw, c, v);
            rht16_unscaled(v, mask);
            mu = __builtin_fmaxf(mu, absmax16(v));
        }
        // rounding is monotonic: the max of the scaled values is the scaled max
        m = max(m, __float_as_uint(mu * 0.25f));
    }
    }
    m = wave_max_u32(m);
    __shared__ uint32_t red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) merge_amax(amax_bits, max(max(red[0], red[1]), max(red[2], red[3])));
}

// One pass over a tokens x channels matrix: max |x| and max |RHT(x)| (the
// transform nvfp4_rht_quantize applies), for callers that quantise the same
// tensor both ways.
__global__ __launch_bounds__(256) void k_amax_dual(const uint16_t* __restrict__ x, int64_t tokens,
                                                   int64_t channels, int64_t ld, uint32_t mask,
                                                   uint32_t* __restrict__ amax_bits,
                                                   uint32_t* __restrict__ amax_rht_bits)
{
    const int cg = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int64_t bch = (channels + kAmCh - 1) / kAmCh, btok = (tokens + kAmTok - 1) / kAmTok;
    uint32_t m = 0u, mr = 0u;
    for (int64_t bt = blockIdx.x; bt < bch * btok; bt += gridDim.x) {
    const int64_t ch0 = (bt % bch) * kAmCh + cg * 8;
    const int64_t tok0 = (bt / bch) * kAmTok + j * 16;
    if (ch0 < channels && tok0 < tokens) {
        uint4 raw[16];
        load_rht_raw(x, ld, tok0, ch0, raw);
#pragma unroll
        for (int i = 0; i < 16; ++i) m = max(m, absmax8(raw[i]));
        float mu = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float v[16];
            unpack_channel(raw, c, v);
            rht16_unscaled(v, mask);
            mu = __builtin_fmaxf(mu, absmax16(v));
        }
        // rounding is monotonic: the max of the scaled values is the scaled max
        mr = max(mr, __float_as_uint(mu * 0.25f));
    }
    }
    m = wave_max_u32(m);
    mr = wave_max_u32(mr);
    __shared__ uint32_t red[2][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red[0][wave] = m;
        red[1][wave] = mr;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        merge_amax(amax_bits, max(max(red[0][0], red[0][1]), max(red[0][2], red[0][3])) << 16);
        merge_amax(amax_rht_bits, max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3])));
    }
}

template <bool kSR>
__global__ __launch_bounds__(256) void k_rht_quant(
    const uint16_t* __restrict__ x, int64_t tokens, int64_t channels, int64_t ld, uint32_t mask,
    const float* __restrict__ amax_src, uint64_t seed, uint8_t* __restrict__ codes,
    int64_t ld_codes, bool il, uint8_t* __restrict__ scales, int64_t ld_scales,
    float* __restrict__ amax_out, float* __restrict__ s_enc_out)
{
    __shared__ uint2 scodes[kRhtCh][17];    // [channel][chunk], padded
    __shared__ uint8_t sscale[kRhtCh][16];  // [channel][chunk]

    const int cg = threadIdx.x & 15, j = threadIdx.x >> 4;
    const int64_t chb = (int64_t)blockIdx.x * kRhtCh, tokb = (int64_t)blockIdx.y * kRhtTok;
    const int64_t ch0 = chb + cg * 8;
    const int64_t tok0 = tokb + j * 16;
    const float amax = *amax_src;
    const float s_enc = tensor_scale(amax);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        *amax_out = amax;
        *s_enc_out = s_enc;
    }
    if (ch0 < channels && tok0 < tokens) {
        uint4 raw[16];
        load_rht_raw(x, ld, tok0, ch0, raw);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float v[16];
            unpack_channel(raw, c, v);
            rht16(v, mask);
            const uint32_t sb = block_scale(absmax16(v), s_enc);
            const float f = block_factor(sb, s_enc);
            uint2 pk;
            if constexpr (kSR)
                pk = encode16_sr(v, f, seed, (uint64_t)((ch0 + c) * tokens + tok0) >> 3);
            else
                pk = encode16_rne(v, f);
            scodes[cg * 8 + c][j] = pk;
            sscale[cg * 8 + c][j] = (uint8_t)sb;
        }
    }
    __syncthreads();
    // 128 channel rows x 16 chunks of 8 code bytes; 16 consecutive threads
    // write one row's 128 contiguous bytes.
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int idx = it * 256 + threadIdx.x;
        const int row = idx >> 4, q = idx & 15;
        const int64_t ch = chb + row, tk = tokb + q * 16;
        if (ch < channels && tk < tokens) {
            *reinterpret_cast<uint2*>(codes + code_offset(ch, tk >> 1, ld_codes, il)) = scodes[row][q];
            scales[ch * ld_scales + (tk >> 4)] = sscale[row][q];
        }
    }
}

// ---------------------------------------------------------------------------
// Dual quantiser: one read of a tokens x channels matrix yields both its 1x16
// quantisation along the channels (the fprop or dgrad operand) and the
// RHT-transposed 1x16 quantisation along the tokens (the wgrad operand), with
// the same codes as k_quant_1x16 and k_rht_quant.  Tile and thread map are
// k_rht_quant's; a row block's 16 channels are the 8 + 8 held by lanes 2q and
// 2q + 1 of one wave, so its amax is one lane shuffle.
// ---------------------------------------------------------------------------

// 8 values times f -> 4 packed bytes (RNE)
__device__ __forceinline__ uint32_t encode8_rne(const float (&v)[8], float f)
{
    uint32_t w = 0u;
    w = e2m1_rne_pk<0>(w, v[0] * f, v[1] * f);
    w = e2m1_rne_pk<1>(w, v[2] * f, v[3] * f);
    w = e2m1_rne_pk<2>(w, v[4] * f, v[5] * f);
    w = e2m1_rne_pk<3>(w, v[6] * f, v[7] * f);
    return w;
}

// 8 values times f, stochastically rounded with the draws of elements
// 8*g8 .. 8*g8+7 (one Philox block) -> 4 packed bytes
__device__ __forceinline__ uint32_t encode8_sr(const float (&v)[8], float f, uint64_t seed,
                                               uint64_t g8)
{
    const Draws8 d = sr_draws8(seed, g8);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[i] * f;
    return e2m1_sr8(y, d.w);
}

// (three waves per SIMD requested: the compiler's default schedule holds
// 186 VGPRs for SR, two waves; at 168 the SR encode runs 6 % faster)
template <bool kSR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_dual_quant(
    const uint16_t* __restrict__ x, int64_t tokens, int64_t channels, int64_t ld, uint32_t mask,
    const float* __restrict__ amax_src, const float* __restrict__ amax_rht_src, uint64_t seed,
    uint64_t seed_rht, QOut o, QOut o_rht)
{
    __shared__ uint2 scodes[kRhtCh][17];    // transposed codes [channel][chunk], padded
    __shared__ uint8_t sscale[kRhtCh][16];  // [channel][chunk]

    const int cg = threadIdx.x & 15, j = threadIdx.x >> 4;
    const int64_t chb = (int64_t)blockIdx.x * kRhtCh, tokb = (int64_t)blockIdx.y * kRhtTok;
    const int64_t ch0 = chb + cg * 8;
    const int64_t tok0 = tokb + j * 16;
    const float amax = *amax_src, amax_r = *amax_rht_src;
    const float s_enc = tensor_scale(amax), s_enc_r = tensor_scale(amax_r);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        *o.amax = amax;
        *o.s_enc = s_enc;
        *o_rht.amax = amax_r;
        *o_rht.s_enc = s_enc_r;
    }
    // channels is a multiple of 16, so both lanes of a row block are valid
    // or neither is, and the shuffle partner is always active.
    if (ch0 < channels && tok0 < tokens) {
        uint4 raw[16];
        load_rht_raw(x, ld, tok0, ch0, raw);

        // row-wise blocks: token tok0 + i, channels ch0 .. ch0 + 7 of this lane
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t tok = tok0 + i;
            const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
            float v[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                v[2 * k] = bf16_lo(w[k]);
                v[2 * k + 1] = bf16_hi(w[k]);
            }
            uint32_t mb = absmax8(raw[i]) << 16;  // fp32 bits of the lane's max |x|
            mb = max(mb, (uint32_t)__shfl_xor((int)mb, 1, 64));
            const uint32_t sb = block_scale(__uint_as_float(mb), s_enc);
            const float f = block_factor(sb, s_enc);
            uint32_t pk;
            if constexpr (kSR)
                pk = encode8_sr(v, f, seed, (uint64_t)(tok * channels + ch0) >> 3);
            else
                pk = encode8_rne(v, f);
            *reinterpret_cast<uint32_t*>(o.codes + code_offset(tok, ch0 >> 1, o.ld_codes, o.il)) = pk;
            if ((cg & 1) == 0) o.scales[tok * o.ld_scales + (ch0 >> 4)] = (uint8_t)sb;
        }

        // transformed blocks: channel ch0 + c, tokens tok0 .. tok0 + 15
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float v[16];
            unpack_channel(raw, c, v);
            rht16(v, mask);
            const uint32_t sb = block_scale(absmax16(v), s_enc_r);
            const float f = block_factor(sb, s_enc_r);
            uint2 pk;
            if constexpr (kSR)
                pk = encode16_sr(v, f, seed_rht, (uint64_t)((ch0 + c) * tokens + tok0) >> 3);
            else
                pk = encode16_rne(v, f);
            scodes[cg * 8 + c][j] = pk;
            sscale[cg * 8 + c][j] = (uint8_t)sb;
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int idx = it * 256 + threadIdx.x;
        const int row = idx >> 4, q = idx & 15;
        const int64_t ch = chb + row, tk = tokb + q * 16;
        if (ch < channels && tk < tokens) {
            *reinterpret_cast<uint2*>(o_rht.codes + code_offset(ch, tk >> 1, o_rht.ld_codes, o_rht.il)) = scodes[row][q];
            o_rht.scales[ch * o_rht.ld_scales + (tk >> 4)] = sscale[row][q];
        }
    }
}

// ---------------------------------------------------------------------------
// Sized random Hadamard transforms (1, 4, 16 or 64 points) for the size
// ablation of the wgrad operands.  Same tile and thread map as k_rht_quant
// (a thread: 16 tokens x 8 channels); a 64-point chunk spans the lanes
// t, t ^ 16, t ^ 32, t ^ 48 of one wave, whose last two butterfly stages
// (strides 16 and 32) exchange values with lane shuffles.  Size 1 is the
// plain transposing quantiser (no transform) -- the baseline of the study.
// The transform: signs, butterfly strides 1 .. D/2 (each sum and difference
// rounded to fp32, in that order), then the exact normalisation 2^-(log2 D/2).
// ---------------------------------------------------------------------------

template <int D>
__device__ __forceinline__ void rht_sized(float (&v)[16], uint64_t signs, int j)
{
    // sign of token i of this lane's chunk: bit (16 j + i) mod D
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int bit = D >= 16 ? (16 * (j & (D / 16 - 1)) + i) : (i & (D - 1));
        v[i] = __uint_as_float(__float_as_uint(v[i]) ^ ((uint32_t)((signs >> bit) & 1u) << 31));
    }
#pragma unroll
    for (int h = 1; h < (D < 16 ? D : 16); h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
                const float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    if constexpr (D == 64) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {  // strides 16 and 32 tokens: partner chunk j ^ (1 << s)
            const bool upper = (j >> s) & 1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float o = __shfl_xor(v[i], 16 << s, 64);
                v[i] = upper ? o - v[i] : v[i] + o;
            }
        }
    }
    const float norm = D == 64 ? 0.125f : (D == 16 ? 0.25f : (D == 4 ? 0.5f : 1.0f));
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= norm;
}

template <int D>
__global__ __launch_bounds__(256) void k_rhtd_amax(const uint16_t* __restrict__ x, int64_t tokens,
                                                   int64_t channels, int64_t ld, uint64_t signs,
                                                   uint32_t* __restrict__ amax_bits)
{
    const int cg = threadIdx.x & 15, j = threadIdx.x >> 4;
    const int64_t bch = (channels + kRhtCh - 1) / kRhtCh, btok = (tokens + kRhtTok - 1) / kRhtTok;
    uint32_t m = 0u;
    for (int64_t bt = blockIdx.x; bt < bch * btok; bt += gridDim.x) {
        const int64_t ch0 = (bt % bch) * kRhtCh + cg * 8;
        const int64_t tok0 = (bt / bch) * kRhtTok + j * 16;
        // tokens is a multiple of 16 and of D: a D-token chunk is valid as a
        // whole, so the shuffle partners of a valid lane are valid
        if (ch0 < channels && tok0 < tokens) {
            uint4 raw[16];
            load_rht_raw(x, ld, tok0, ch0, raw);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                float v[16];
                unpack_channel(raw, c, v);
                rht_sized<D>(v, signs, j);
                m = max(m, __float_as_uint(absmax16(v)));
            }
        }
    }
    m = wave_max_u32(m);
    __shared__ uint32_t red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) merge_amax(amax_bits, max(max(red[0], red[1]), max(red[2], red[3])));
}

template <bool kSR, int D>
__global__ __launch_bounds__(256) void k_rhtd_quant(
    const uint16_t* __restrict__ x, int64_t tokens, int64_t channels, int64_t ld, uint64_t signs,
    const float* __restrict__ amax_src, uint64_t seed, uint8_t* __restrict__ codes,
    int64_t ld_codes, bool il, uint8_t* __restrict__ scales, int64_t ld_scales,
    float* __restrict__ amax_out, float* __restrict__ s_enc_out)
{
    __shared__ uint2 scodes[kRhtCh][17];
    __shared__ uint8_t sscale[kRhtCh][16];

    const int cg = threadIdx.x & 15, j = threadIdx.x >> 4;
    const int64_t chb = (int64_t)blockIdx.x * kRhtCh, tokb = (int64_t)blockIdx.y * kRhtTok;
    const int64_t ch0 = chb + cg * 8;
    const int64_t tok0 = tokb + j * 16;
    const float amax = *amax_src;
    const float s_enc = tensor_scale(amax);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        *amax_out = amax;
        *s_enc_out = s_enc;
    }
    if (ch0 < channels && tok0 < tokens) {
        uint4 raw[16];
        load_rht_raw(x, ld, tok0, ch0, raw);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float v[16];
            unpack_channel(raw, c, v);
            rht_sized<D>(v, signs, j);
            const uint32_t sb = block_scale(absmax16(v), s_enc);
            const float f = block_factor(sb, s_enc);
            uint2 pk;
            if constexpr (kSR)
                pk = encode16_sr(v, f, seed, (uint64_t)((ch0 + c) * tokens + tok0) >> 3);
            else
                pk = encode16_rne(v, f);
            scodes[cg * 8 + c][j] = pk;
            sscale[cg * 8 + c][j] = (uint8_t)sb;
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int idx = it * 256 + threadIdx.x;
        const int row = idx >> 4, q = idx & 15;
        const int64_t ch = chb + row, tk = tokb + q * 16;
        if (ch < channels && tk < tokens) {
            *reinterpret_cast<uint2*>(codes + code_offset(ch, tk >> 1, ld_codes, il)) = scodes[row][q];
            scales[ch * ld_scales + (tk >> 4)] = sscale[row][q];
        }
    }
}

// ---------------------------------------------------------------------------
// MXFP4 quantisers (the comparison format: 32-element blocks, one UE8M0
// scale each, no tensor scale).  Shared exponent e = floor(log2(amax_b)) - 2
// clamped to [-127, 127]; from the fp32 (or bf16) exponent field E of amax_b
// that is max(E - 129, -127) (E = 0 for zero and subnormal maxima), so the
// scale byte is max(E - 2, 0) and the element factor 2^-e has the fp32
// exponent field min(256 - E, 254).
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t E) { return E > 2u ? E - 2u : 0u; }

__device__ __forceinline__ float mx_factor(uint32_t E)
{
    return __uint_as_float(min(256u - E, 254u) << 23);
}

// Blocks of 32 along the rows of x (rows x cols, cols a multiple of 32): one
// thread per block (four 16-byte loads, a 16-byte code store, a scale byte).
template <bool kSR>
__global__ __launch_bounds__(256) void k_mx_quant_rows(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ scales,
    int64_t ld_scales)
{
    const int64_t nb = cols >> 5;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= rows * nb) return;
    const int64_t r = t / nb;
    const int64_t b = t - r * nb;
    const uint4* src = reinterpret_cast<const uint4*>(x + r * ld + b * 32);
    const uint4 q[4] = {ld_stream(src), ld_stream(src + 1), ld_stream(src + 2), ld_stream(src + 3)};
    const uint32_t mb = max(max(absmax8(q[0]), absmax8(q[1])), max(absmax8(q[2]), absmax8(q[3])));
    const uint32_t E = (mb >> 7) & 0xFFu;  // bf16 exponent field of the block amax
    const float f = mx_factor(E);
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = bf16_lo(w[k]);
            v[2 * k + 1] = bf16_hi(w[k]);
        }
        if constexpr (kSR)
            pk[j] = encode8_sr(v, f, seed, (uint64_t)(r * cols + b * 32 + 8 * j) >> 3);
        else
            pk[j] = encode8_rne(v, f);
    }
    *reinterpret_cast<uint4*>(codes + r * ld_codes + b * 16) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    scales[r * ld_scales + b] = (uint8_t)mx_scale_byte(E);
}

// The transposed matrix (channels x tokens), blocks of 32 along the tokens,
// optionally after the 16-point RHT of every 16-token chunk.  Tile and
// thread map are k_rht_quant's; a block's two 16-token chunks are held by
// lanes t and t ^ 16 of one wave, so its amax is one lane shuffle.
template <bool kSR, bool kRHT>
__global__ __launch_bounds__(256) void k_mx_quant_cols(
    const uint16_t* __restrict__ x, int64_t tokens, int64_t channels, int64_t ld, uint32_t mask,
    uint64_t seed, uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ scales,
    int64_t ld_scales)
{
    __shared__ uint2 scodes[kRhtCh][17];   // [channel][16-token chunk], padded
    __shared__ uint8_t sscale[kRhtCh][8];  // [channel][32-token block]

    const int cg = threadIdx.x & 15, j = threadIdx.x >> 4;
    const int64_t chb = (int64_t)blockIdx.x * kRhtCh, tokb = (int64_t)blockIdx.y * kRhtTok;
    const int64_t ch0 = chb + cg * 8;
    const int64_t tok0 = tokb + j * 16;
    // tokens is a multiple of 32: both chunks of a block are valid or neither
    if (ch0 < channels && tok0 < tokens) {
        uint4 raw[16];
        load_rht_raw(x, ld, tok0, ch0, raw);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float v[16];
            unpack_channel(raw, c, v);
            if constexpr (kRHT) rht16(v, mask);
            uint32_t mb = __float_as_uint(absmax16(v));
            mb = max(mb, (uint32_t)__shfl_xor((int)mb, 16, 64));
            const uint32_t E = mb >> 23;
            const float f = mx_factor(E);
            uint2 pk;
            if constexpr (kSR)
                pk = encode16_sr(v, f, seed, (uint64_t)((ch0 + c) * tokens + tok0) >> 3);
            else
                pk = encode16_rne(v, f);
            scodes[cg * 8 + c][j] = pk;
            if ((j & 1) == 0) sscale[cg * 8 + c][j >> 1] = (uint8_t)mx_scale_byte(E);
        }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int idx = it * 256 + threadIdx.x;
        const int row = idx >> 4, q = idx & 15;
        const int64_t ch = chb + row, tk = tokb + q * 16;
        if (ch < channels && tk < tokens) {
            *reinterpret_cast<uint2*>(codes + ch * ld_codes + (tk >> 1)) = scodes[row][q];
            if ((q & 1) == 0) scales[ch * ld_scales + (tk >> 5)] = sscale[row][q >> 1];
        }
    }
}

// max |RHT(x)| with the transform on every aligned 16-element chunk of the
// rows (fprop / dgrad ablation): one chunk per thread, grid-stride.
__global__ __launch_bounds__(256) void k_amax_rows_rht(const uint16_t* __restrict__ x, int64_t rows,
                                                       int64_t cols, int64_t ld, uint32_t mask,
                                                       uint32_t* __restrict__ amax_bits)
{
    const int64_t nb = cols >> 4;
    uint32_t m = 0u;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < rows * nb; t += stride) {
        const int64_t r = t / nb, b = t - r * nb;
        const uint4* src = reinterpret_cast<const uint4*>(x + r * ld + b * 16);
        float v[16];
        unpack16(ld_stream(src), ld_stream(src + 1), v);
        rht16_unscaled(v, mask);
        // rounding is monotonic: the max of the scaled values is the scaled max
        m = max(m, __float_as_uint(absmax16(v) * 0.25f));
    }
    m = wave_max_u32(m);
    __shared__ uint32_t red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) merge_amax(amax_bits, max(max(red[0], red[1]), max(red[2], red[3])));
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static int grid_for(int64_t work, int64_t per_block, int64_t cap)
{
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    return (int)(g < cap ? g : cap);
}

// Threads of a k_quant_1x16 launch: a workgroup of 256 per 4 rows x 64 blocks.
static int64_t quant_1x16_threads(int64_t rows, int64_t cols)
{
    return ((rows + 3) / 4) * (((cols >> 4) + 63) / 64) * 256;
}

void launch_amax_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, float* amax,
                      hipStream_t s)
{
    uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, s, bits);
    const int64_t nvec = rows * (cols >> 3);
    if (nvec == 0) return;
    if (ld == cols) {
        hipLaunchKernelGGL(k_amax_flat, dim3(grid_for(nvec, 256 * kFlatLoads, kFlatGrid)), dim3(256), 0, s,
                           reinterpret_cast<const uint4*>(x), nvec, bits);
    } else {
        hipLaunchKernelGGL(k_amax_rows, dim3(grid_for(nvec, 256, 4096)), dim3(256), 0, s, x, rows,
                           cols, ld, bits);
    }
}

void launch_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int block,
                  int rounding, uint64_t seed, const float* amax_src, const QOut& o, hipStream_t s)
{
    const bool sr = rounding == 1;
    if (rows == 0 || cols == 0) {
        hipLaunchKernelGGL(k_publish, dim3(1), dim3(1), 0, s, amax_src, o.amax, o.s_enc);
        return;
    }
    if (block == 0) {
        dim3 g(grid_for(quant_1x16_threads(rows, cols), 256, INT32_MAX));
        if (sr)
            hipLaunchKernelGGL(k_quant_1x16<true>, g, dim3(256), 0, s, x, rows, cols, ld, amax_src,
                               seed, o.codes, o.ld_codes, o.il, o.scales, o.ld_scales, o.amax, o.s_enc);
        else
            hipLaunchKernelGGL(k_quant_1x16<false>, g, dim3(256), 0, s, x, rows, cols, ld, amax_src,
                               seed, o.codes, o.ld_codes, o.il, o.scales, o.ld_scales, o.amax, o.s_enc);
    } else if (o.il) {
        const int64_t tiles = ((cols + kW3Cols - 1) / kW3Cols) * ((rows + 16 * kW3Waves - 1) / (16 * kW3Waves));
        dim3 g(grid_for(tiles, 1, INT32_MAX));
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, g, dim3(64 * kW3Waves), 0, s, x, rows, cols, ld, amax_src, seed,
                               o.codes, o.ld_codes, o.scales, o.ld_scales, o.codes_t, o.ld_codes_t,
                               o.scales_t, o.ld_scales_t, o.amax, o.s_enc);
        };
        sr ? go(k_quant_16x16_il<true>) : go(k_quant_16x16_il<false>);
    } else {
        dim3 g((unsigned)((cols + kW2Cols - 1) / kW2Cols), (unsigned)((rows + kW2Rows - 1) / kW2Rows));
        if (sr)
            hipLaunchKernelGGL(k_quant_16x16<true>, g, dim3(kW2TC * kW2RG), 0, s, x, rows, cols, ld,
                               amax_src, seed, o.codes, o.ld_codes, o.il, o.scales, o.ld_scales,
                               o.codes_t, o.ld_codes_t, o.scales_t, o.ld_scales_t, o.amax, o.s_enc);
        else
            hipLaunchKernelGGL(k_quant_16x16<false>, g, dim3(kW2TC * kW2RG), 0, s, x, rows, cols, ld,
                               amax_src, seed, o.codes, o.ld_codes, o.il, o.scales, o.ld_scales,
                               o.codes_t, o.ld_codes_t, o.scales_t, o.ld_scales_t, o.amax, o.s_enc);
    }
}

void launch_rht_amax(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld,
                     uint32_t mask, float* amax, hipStream_t s)
{
    uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, s, bits);
    if (tokens == 0 || channels == 0) return;
    dim3 g(grid_for(((channels + kAmCh - 1) / kAmCh) * ((tokens + kAmTok - 1) / kAmTok), 1, kAmaxGrid));
    hipLaunchKernelGGL(k_rht_amax, g, dim3(256), 0, s, x, tokens, channels, ld, mask, bits);
}

void launch_amax_dual(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld,
                      uint32_t mask, float* amax, float* amax_rht, hipStream_t s)
{
    uint32_t* b0 = reinterpret_cast<uint32_t*>(amax);
    uint32_t* b1 = reinterpret_cast<uint32_t*>(amax_rht);
    hipLaunchKernelGGL(k_zero_u32x2, dim3(1), dim3(1), 0, s, b0, b1);
    if (tokens == 0 || channels == 0) return;
    dim3 g(grid_for(((channels + kAmCh - 1) / kAmCh) * ((tokens + kAmTok - 1) / kAmTok), 1, kAmaxGrid));
    hipLaunchKernelGGL(k_amax_dual, g, dim3(256), 0, s, x, tokens, channels, ld, mask, b0, b1);
}

void launch_rht_quant(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld,
                      uint32_t mask, int rounding, uint64_t seed, const float* amax_src,
                      const QOut& o, hipStream_t s)
{
    if (tokens == 0 || channels == 0) {
        hipLaunchKernelGGL(k_publish, dim3(1), dim3(1), 0, s, amax_src, o.amax, o.s_enc);
        return;
    }
    dim3 g((unsigned)((channels + kRhtCh - 1) / kRhtCh), (unsigned)((tokens + kRhtTok - 1) / kRhtTok));
    if (rounding == 1)
        hipLaunchKernelGGL(k_rht_quant<true>, g, dim3(256), 0, s, x, tokens, channels, ld, mask,
                           amax_src, seed, o.codes, o.ld_codes, o.il, o.scales, o.ld_scales, o.amax,
                           o.s_enc);
    else
        hipLaunchKernelGGL(k_rht_quant<false>, g, dim3(256), 0, s, x, tokens, channels, ld, mask,
                           amax_src, seed, o.codes, o.ld_codes, o.il, o.scales, o.ld_scales, o.amax,
                           o.s_enc);
}

void launch_dual_quant(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld,
                       uint32_t mask, int rounding, uint64_t seed, uint64_t seed_rht,
                       const float* amax_src, const float* amax_rht_src, const QOut& o,
                       const QOut& o_rht, hipStream_t s)
{
    if (tokens == 0 || channels == 0) {
        hipLaunchKernelGGL(k_publish, dim3(1), dim3(1), 0, s, amax_src, o.amax, o.s_enc);
        hipLaunchKernelGGL(k_publish, dim3(1), dim3(1), 0, s, amax_rht_src, o_rht.amax,
                           o_rht.s_enc);
        return;
    }
    dim3 g((unsigned)((channels + kRhtCh - 1) / kRhtCh), (unsigned)((tokens + kRhtTok - 1) / kRhtTok));
    if (rounding == 1)
        hipLaunchKernelGGL(k_dual_quant<true>, g, dim3(256), 0, s, x, tokens, channels, ld, mask,
                           amax_src, amax_rht_src, seed, seed_rht, o, o_rht);
    else
        hipLaunchKernelGGL(k_dual_quant<false>, g, dim3(256), 0, s, x, tokens, channels, ld, mask,
                           amax_src, amax_rht_src, seed, seed_rht, o, o_rht);
}

void launch_mx_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int mode,
                     uint32_t mask, int rounding, uint64_t seed, const QOut& o, hipStream_t s)
{
    if (rows == 0 || cols == 0) return;
    const bool sr = rounding == 1;
    if (mode == 0) {
        dim3 g(grid_for(rows * (cols >> 5), 256, INT32_MAX));
        if (sr)
            hipLaunchKernelGGL(k_mx_quant_rows<true>, g, dim3(256), 0, s, x, rows, cols, ld, seed,
                               o.codes, o.ld_codes, o.scales, o.ld_scales);
        else
            hipLaunchKernelGGL(k_mx_quant_rows<false>, g, dim3(256), 0, s, x, rows, cols, ld, seed,
                               o.codes, o.ld_codes, o.scales, o.ld_scales);
        return;
    }
    dim3 g((unsigned)((cols + kRhtCh - 1) / kRhtCh), (unsigned)((rows + kRhtTok - 1) / kRhtTok));
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, g, dim3(256), 0, s, x, rows, cols, ld, mask, seed, o.codes,
                           o.ld_codes, o.scales, o.ld_scales);
    };
    if (mode == 1)
        sr ? go(k_mx_quant_cols<true, false>) : go(k_mx_quant_cols<false, false>);
    else
        sr ? go(k_mx_quant_cols<true, true>) : go(k_mx_quant_cols<false, true>);
}

void launch_rhtd_amax(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld, int size,
                      uint64_t signs, float* amax, hipStream_t s)
{
    uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, s, bits);
    if (tokens == 0 || channels == 0) return;
    dim3 g(grid_for(((channels + kRhtCh - 1) / kRhtCh) * ((tokens + kRhtTok - 1) / kRhtTok), 1, kAmaxGrid));
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, g, dim3(256), 0, s, x, tokens, channels, ld, signs, bits); };
    switch (size) {
        case 1: go(k_rhtd_amax<1>); break;
        case 4: go(k_rhtd_amax<4>); break;
        case 16: go(k_rhtd_amax<16>); break;
        default: go(k_rhtd_amax<64>); break;
    }
}

void launch_rhtd_quant(const uint16_t* x, int64_t tokens, int64_t channels, int64_t ld, int size,
                       uint64_t signs, int rounding, uint64_t seed, const float* amax_src,
                       const QOut& o, hipStream_t s)
{
    if (tokens == 0 || channels == 0) {
        hipLaunchKernelGGL(k_publish, dim3(1), dim3(1), 0, s, amax_src, o.amax, o.s_enc);
        return;
    }
    dim3 g((unsigned)((channels + kRhtCh - 1) / kRhtCh), (unsigned)((tokens + kRhtTok - 1) / kRhtTok));
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, g, dim3(256), 0, s, x, tokens, channels, ld, signs, amax_src, seed,
                           o.codes, o.ld_codes, o.il, o.scales, o.ld_scales, o.amax, o.s_enc);
    };
    const bool sr = rounding == 1;
    switch (size) {
        case 1: sr ? go(k_rhtd_quant<true, 1>) : go(k_rhtd_quant<false, 1>); break;
        case 4: sr ? go(k_rhtd_quant<true, 4>) : go(k_rhtd_quant<false, 4>); break;
        case 16: sr ? go(k_rhtd_quant<true, 16>) : go(k_rhtd_quant<false, 16>); break;
        default: sr ? go(k_rhtd_quant<true, 64>) : go(k_rhtd_quant<false, 64>); break;
    }
}

void launch_amax_rows_rht(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint32_t mask,
                          float* amax, hipStream_t s)
{
    uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
    hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, s, bits);
    const int64_t work = rows * (cols >> 4);
    if (work == 0) return;
    hipLaunchKernelGGL(k_amax_rows_rht, dim3(grid_for(work, 256, 2048)), dim3(256), 0, s, x, rows, cols,
                       ld, mask, bits);
}

void launch_quant_rht_rows(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int block,
                           uint32_t mask, int rounding, uint64_t seed, const float* amax_src,
                           const QOut& o, hipStream_t s)
{
    const bool sr = rounding == 1;
    if (rows == 0 || cols == 0) {
        hipLaunchKernelGGL(k_publish, dim3(1), dim3(1), 0, s, amax_src, o.amax, o.s_enc);
        return;
    }
    if (block == 0) {
        dim3 g(grid_for(quant_1x16_threads(rows, cols), 256, INT32_MAX));
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, g, dim3(256), 0, s, x, rows, cols, ld, amax_src, seed, o.codes,
                               o.ld_codes, o.il, o.scales, o.ld_scales, o.amax, o.s_enc, mask);
        };
        sr ? go(k_quant_1x16<true, true>) : go(k_quant_1x16<false, true>);
    } else {
        dim3 g((unsigned)((cols + kW2Cols - 1) / kW2Cols), (unsigned)((rows + kW2Rows - 1) / kW2Rows));
        auto go = [&](auto kern) {
            hipLaunchKernelGGL(kern, g, dim3(kW2TC * kW2RG), 0, s, x, rows, cols, ld, amax_src, seed, o.codes,
                               o.ld_codes, o.il, o.scales, o.ld_scales, o.codes_t, o.ld_codes_t, o.scales_t,
                               o.ld_scales_t, o.amax, o.s_enc, mask);
        };
        sr ? go(k_quant_16x16<true, true>) : go(k_quant_16x16<false, true>);
    }
}

}  // namespace nvfp4
