// nvfp4_device.hpp -- device-side number formats and helpers for gfx950.
//
// Format and recipe: "Pretraining Large Language Models with NVFP4"
// (gist.science summary), Technische Zusammenfassung 2.A (E2M1 elements in
// 16-element blocks, E4M3 block scale, FP32 tensor scale) and 2.B.4 (RNE for
// activations and weights, stochastic rounding for gradients).
//
// All fp32 arithmetic here is IEEE binary32 with round-to-nearest-even; the
// library is built with -ffp-contract=off so that no multiply-add is fused,
// and fp32 division is the correctly rounded one (the HIP default).  The
// quantised codes are integer decisions taken in fp32 and must not depend on
// the compiler's choices.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kFltMax = 3.40282346638528859812e+38f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((vector_size(8)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Where byte j of code row r lies in a codes buffer with rows ld bytes long.
// Row-major: r * ld + j.  Interleaved (il): rows in groups of 4, each
// 128-byte piece holding 32 bytes (64 codes, one K step of the GEMMs) of the
// 4 rows in turn, so that a K step of 4 rows is one whole cache line:
// (r / 4) * 4 * ld + (j / 32) * 128 + (r % 4) * 32 + j % 32, ld a multiple of
// 32.  A write of up to 32 aligned bytes stays inside one piece.
__device__ __forceinline__ int64_t code_offset(int64_t r, int64_t j, int64_t ld, bool il)
{
    return il ? (r >> 2) * 4 * ld + ((j >> 5) << 7) + ((r & 3) << 5) + (j & 31) : r * ld + j;
}

// |bf16| ordering equals the unsigned ordering of the 15 magnitude bits.
__device__ __forceinline__ uint32_t bf16_absmax2(uint32_t w)
{
    return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

// The output scale of a GEMM over two NVFP4 operands: the product of their
// FP32 tensor decode scales d = 1 / s_enc (format: FP32 per-tensor scale).
// The product is returned as am * 2^e: when d_a * d_b is a normal fp32
// number, am is that product and e = 0; below fp32's normal range (both
// tensor maxima tiny, amax_a * amax_b < ~8.5e-32) am is the rounded product
// of the two significands and e the sum of the exponents, so that
// out = ldexp(acc * am, e) keeps 24 significant bits wherever the output
// itself is a normal number.  A single fp32 product would be subnormal there
// and lose precision (or reach zero) although every factor and every output
// is normal.
__device__ __forceinline__ void output_scale(float s_enc_a, float s_enc_b, float& am, int& e)
{
    const float da = 1.0f / s_enc_a, db = 1.0f / s_enc_b;
    am = da * db;
    e = 0;
    if (!(am >= 1.17549435e-38f)) {  // below FLT_MIN: keep the exponent apart
        int ea, eb;
        const float ma = __builtin_frexpf(da, &ea), mb = __builtin_frexpf(db, &eb);
        am = ma * mb;  // in [0.25, 1): normal
        e = ea + eb;
    }
}

// Tensor encode scale: 2688 / amax (2688 = 6 * 448 maps the tensor amax to
// the largest E2M1 value under the largest E4M3 scale); 1 for amax = 0,
// FLT_MAX when the quotient overflows.
__device__ __forceinline__ float tensor_scale(float amax)
{
    if (amax == 0.0f) return 1.0f;
    float s = 2688.0f / amax;
    return (s <= kFltMax) ? s : kFltMax;
}

// Non-negative fp32 -> E4M3 byte, round to nearest even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode(float t)
{
    if (!(t > 0.0f)) return 0u;
    if (t >= 448.0f) return 0x7Eu;
    if (t < 0.015625f) return (uint32_t)__builtin_rintf(t * 512.0f);  // k * 2^-9, k = 8 is 0x08
    uint32_t u = __float_as_uint(t);
    u += 0x7FFFFu + ((u >> 20) & 1u);   // keep 3 mantissa bits, ties to even
    return (u >> 20) - (120u << 3);     // rebias the exponent from 127 to 7
}

// E4M3 byte (non-negative, not NaN) -> fp32.
__device__ __forceinline__ float e4m3_decode(uint32_t b)
{
    return (b & 0x78u) ? __uint_as_float((b << 20) + (120u << 23)) : (float)b * 0.001953125f;
}

// Block scale byte from the block amax and the tensor scale.
__device__ __forceinline__ uint32_t block_scale(float amax_b, float s_enc)
{
    float t = (amax_b / 6.0f) * s_enc;
    return e4m3_encode(t);
}

// Per-element factor s_enc / S_b (0 for a zero scale, clamped to FLT_MAX).
__device__ __forceinline__ float block_factor(uint32_t sb, float s_enc)
{
    float S = e4m3_decode(sb);
    if (!(S > 0.0f)) return 0.0f;
    float f = s_enc / S;
    return (f <= kFltMax) ? f : kFltMax;
}

// Two fp32 values -> two E2M1 codes (RNE, saturating, sign of zero kept)
// written into byte `sel` of `old`; y0 goes to the low nibble.  The hardware
// conversion with a unit scale is exactly E2M1 round-to-nearest-even.
template <int sel>
__device__ __forceinline__ uint32_t e2m1_rne_pk(uint32_t old, float y0, float y1)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y0, y1, 1.0f, sel);
}

// Stochastic rounding onto the E2M1 grid with a 16-bit draw u16 per value:
// with lo the grid point at or below |y| and g the gap above it, round up
// iff u16 < P = trunc((|y| - lo) / g * 2^16); |y| >= 6 gives 6; the sign is
// kept (also of zero).
//
// gfx950's v_cvt_scalef32_sr_pk_fp4_f32 (unit scale) rounds the first value
// of its pair up iff bits [31:16] of its random operand plus the top 16 bits
// of the fraction it discards carry out of 16 bits; with the operand's low
// 16 bits zero nothing carries in from below.  The operand
// (0xFFFF - u16) << 16 therefore gives exactly the rule above:
// u16 < P  <=>  (0xFFFF - u16) + P >= 2^16.  The pair's second value reads
// bits [30:15], which overlap, so every value gets an instruction of its
// own (the same value in both slots).  Each conversion writes byte 0 of its
// own result, code in the low nibble; the other bytes are not relied on
// (the compiler does not carry the destination's old bytes through the
// byte-select forms of this instruction).
__device__ __forceinline__ uint32_t e2m1_sr_conv(float y, uint32_t rnd)
{
    const float2_t v = {y, y};
    return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, v, rnd, 1.0f, 0);
}

// Byte 0 of a, b, c, d -> bytes 0, 1, 2, 3.
__device__ __forceinline__ uint32_t gather_byte0(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Eight values with their draws (Draws8 layout: element 2k takes the low
// half of word k, element 2k+1 the high half) -> 8 codes, low nibble first.
__device__ __forceinline__ uint32_t e2m1_sr8(const float (&y)[8], const uint32_t (&w)[4])
{
    uint32_t t[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t n = ~w[k];
        t[2 * k] = e2m1_sr_conv(y[2 * k], n << 16);
        t[2 * k + 1] = e2m1_sr_conv(y[2 * k + 1], n & 0xFFFF0000u);
    }
    const uint32_t ev = gather_byte0(t[0], t[2], t[4], t[6]);
    const uint32_t od = gather_byte0(t[1], t[3], t[5], t[7]);
    return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
}

// Philox4x32-10 block function (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11).
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2,
                                              uint32_t& c3, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input xor in one instruction (truth table 0x96)
        uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// The eight 16-bit draws of elements 8*g8 .. 8*g8+7 (counter (g8, 0, 0)).
struct Draws8 {
    uint32_t w[4];
    __device__ __forceinline__ uint32_t get(int j) const { return (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu; }
};

__device__ __forceinline__ Draws8 sr_draws8(uint64_t seed, uint64_t g8)
{
    Draws8 d;
    uint32_t c0 = (uint32_t)g8, c1 = (uint32_t)(g8 >> 32), c2 = 0u, c3 = 0u;
    philox4x32_10(c0, c1, c2, c3, (uint32_t)seed, (uint32_t)(seed >> 32));
    d.w[0] = c0;
    d.w[1] = c1;
    d.w[2] = c2;
    d.w[3] = c3;
    return d;
}

// 16-point random Hadamard transform of v (in place), without the final
// factor 1/4: sign flips from `mask`, then the radix-2 butterfly with strides
// 1, 2, 4, 8 (each sum and difference rounded to fp32).
__device__ __forceinline__ void rht16_unscaled(float (&v)[16], uint32_t mask)
{
#pragma unroll
    for (int i = 0; i < 16; ++i)  // negation as a sign-bit flip (exact, branch-free)
        v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((mask >> i) & 1u) << 31));
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

// The full transform: the butterfly above, then the exact multiplication by
// 1/4.  This fixes the rounding order that the codes depend on.
__device__ __forceinline__ void rht16(float (&v)[16], uint32_t mask)
{
    rht16_unscaled(v, mask);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] *= 0.25f;
}

// Wave-wide max of a non-negative value (as uint bits).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
    return v;
}

}  // namespace nvfp4
