/*
 * nvfp4_oracle.c -- plain CPU oracle for the NVFP4 quantize -> GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the bench's
 * cpu_baseline leg may load this library.  The GPU product path never calls
 * it, shares no code with it, and includes none of its headers.
 *
 * Every step is written out element by element, in IEEE binary32 with
 * round-to-nearest-even and no fused multiply-add (built with
 * -ffp-contract=off, no fast-math), because the quantised codes are integer
 * decisions taken in fp32 and must be reproduced bit for bit.
 *
 * Sources (web pages about NVIDIA's report "Pretraining Large Language Models
 * with NVFP4"):
 *   [P1] "Pretraining Large Language Models with NVFP4" (gist.science summary),
 *        sections "Das Wesentliche" and "Technische Zusammenfassung" (TZ).
 *   [P2] "LLM-Pretraining in 4-Bit: NVIDIA stellt NVFP4-Trainingsansatz vor",
 *        section "Das Wichtigste".
 * The pages fix the recipe (which tensor gets which treatment) but not the
 * arithmetic; each reading taken where they are silent is marked "reading"
 * below.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_SHAPE (-2)
#define ORC_ERR_MODE (-4)

#define ORC_BLOCK_1X16 0
#define ORC_BLOCK_16X16 1
#define ORC_RNE 0
#define ORC_SR 1

/* ------------------------------------------------------------------------ */
/* Number formats.                                                          */
/* ------------------------------------------------------------------------ */

/* bf16 input -> fp32: the bf16 bits are the top half of the fp32 bits. */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/*
 * FP4 element (E2M1).  [P1] TZ 1 and 2.A say only "4-bit floating point";
 * reading: the OCP MX E2M1 layout, 1 sign bit, 2 exponent bits (bias 1),
 * 1 mantissa bit, no Inf/NaN.  Code = sign<<3 | exponent<<1 | mantissa.
 * Exponent 0 is subnormal: value = mantissa * 0.5.
 */
double orc_e2m1_decode(uint8_t code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* Magnitude code of an exactly representable E2M1 magnitude. */
static uint8_t e2m1_mag_code(float v)
{
    /* 2*v is one of 0,1,2,3,4,6,8,12 */
    switch ((int)(v * 2.0f)) {
    case 0: return 0;
    case 1: return 1;
    case 2: return 2;
    case 3: return 3;
    case 4: return 4;
    case 6: return 5;
    case 8: return 6;
    default: return 7; /* 12 */
    }
}

/*
 * Round-to-nearest-even onto the E2M1 grid {0, .5, 1, 1.5, 2, 3, 4, 6}.
 * [P1] TZ 2.B.4: activations and weights use round-to-nearest-even.
 * The grid spacing is 0.5 below 2, 1 on [2,4) and 2 on [4,6]; rounding a/q
 * to the nearest integer with ties to even picks the even code, because on
 * this grid an even multiple of the spacing is an even code.  Magnitudes
 * above 6 saturate to 6 (reading).  The sign is the sign bit of y, so -0
 * gives code 8 (reading).
 */
uint8_t orc_e2m1_encode_rne(float y)
{
    uint8_t s = signbit(y) ? 8 : 0;
    float a = fabsf(y);
    float q = (a < 2.0f) ? 0.5f : (a < 4.0f) ? 1.0f : 2.0f;
    float m = rintf(a / q) * q; /* a/q and the product are exact */
    if (m > 6.0f) m = 6.0f;
    return (uint8_t)(s | e2m1_mag_code(m));
}

/*
 * Stochastic rounding onto the E2M1 grid.  [P1] TZ 2.B.4: gradients are
 * rounded at random to one of the two neighbouring representable values so
 * that the rounding is unbiased.  Reading: with lo = the grid value at or
 * below |y| and g = the grid gap above it, r = (|y| - lo) / g is exact, and
 * the magnitude rounds up to lo + g iff u16 < trunc(r * 2^16), where u16 is
 * a 16-bit uniform draw.  |y| >= 6 saturates to 6.
 */
uint8_t orc_e2m1_encode_sr(float y, uint16_t u16)
{
    uint8_t s = signbit(y) ? 8 : 0;
    float a = fabsf(y);
    if (a >= 6.0f) return (uint8_t)(s | 7);
    float g = (a < 2.0f) ? 0.5f : (a < 4.0f) ? 1.0f : 2.0f;
    float lo = floorf(a / g) * g;
    float r = (a - lo) / g;                /* exact */
    uint32_t P = (uint32_t)(r * 65536.0f); /* exact scaling, then truncation */
    float v = ((uint32_t)u16 < P) ? lo + g : lo;
    return (uint8_t)(s | e2m1_mag_code(v));
}

/*
 * Block scale format E4M3 ([P1] TZ 2.A: block scales are E4M3 rather than
 * UE8M0).  Reading: OCP FP8 E4M3, bias 7, subnormals down to 2^-9, largest
 * finite value 448 (0x7E); 0x7F is NaN and is never produced.
 */
float orc_e4m3_decode(uint8_t b)
{
    int s = (b >> 7) & 1, e = (b >> 3) & 15, m = b & 7;
    float mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) mag = ldexpf((float)m, -9);
    else mag = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -mag : mag;
}

/*
 * Non-negative fp32 -> nearest E4M3 value, ties to even mantissa, values at
 * or above 448 saturate to 448 (the scale never becomes NaN).
 */
uint8_t orc_e4m3_encode_rne_sat(float t)
{
    if (!(t > 0.0f)) return 0;
    if (t >= 448.0f) return 0x7E;
    int e2;
    frexpf(t, &e2);        /* t = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;        /* floor(log2 t) */
    if (E < -6) E = -6;    /* below 2^-6 the spacing stays 2^-9 */
    float quantum = ldexpf(1.0f, E - 3);
    float k = rintf(t / quantum); /* exact division by a power of two */
    float v = k * quantum;
    if (v > 448.0f) v = 448.0f;
    if (v < ldexpf(1.0f, -6)) return (uint8_t)k; /* subnormal: k * 2^-9 */
    frexpf(v, &e2);
    E = e2 - 1;
    int mant = (int)((ldexpf(v, -E) - 1.0f) * 8.0f);
    return (uint8_t)(((E + 7) << 3) | mant);
}

/* ------------------------------------------------------------------------ */
/* Counter-based random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw,  */
/* "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11).                    */
/* ------------------------------------------------------------------------ */

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * c0;
        uint64_t p1 = (uint64_t)M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/*
 * The 16-bit draw for element `idx` (row-major index in the layout of the
 * quantised operand): Philox4x32-10 with key = (low, high 32 bits of seed),
 * counter = (low, high 32 bits of idx/8, 0, 0); element idx%8 takes half
 * (idx%2) of output word (idx%8)/2, low half first.
 */
uint16_t orc_sr_draw(uint64_t seed, uint64_t idx)
{
    uint64_t g8 = idx >> 3;
    uint32_t j = (uint32_t)(idx & 7);
    uint32_t ctr[4] = {(uint32_t)g8, (uint32_t)(g8 >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    return (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
}

/*
 * Sign vector of the random Hadamard transform: bit i set means d_i = -1.
 * Reading: the low 16 bits of word 0 of Philox4x32-10 with key = seed and
 * counter (0, 0, 0, 1); the third counter word 1 never occurs in the
 * stochastic-rounding draws, whose counters end in (0, 0).
 */
uint32_t orc_rht_sign_mask(uint64_t seed)
{
    uint32_t ctr[4] = {0u, 0u, 0u, 1u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    return w[0] & 0xFFFFu;
}

/* ------------------------------------------------------------------------ */
/* Two-level scaling ([P1] TZ 2.A and "Das Wesentliche", trick 2).          */
/* ------------------------------------------------------------------------ */

/*
 * Tensor-level FP32 encode scale.  Reading: s_enc = 2688 / amax with
 * 2688 = 6 * 448 (E2M1 max times E4M3 max), so that the block holding the
 * tensor amax gets the largest E4M3 scale and its largest element the
 * largest E2M1 value.  amax = 0 gives 1; a non-finite quotient gives FLT_MAX.
 */
float orc_tensor_scale(float amax)
{
    if (amax == 0.0f) return 1.0f;
    float s = 2688.0f / amax;
    if (!isfinite(s)) s = FLT_MAX;
    return s;
}

/*
 * E4M3 block scale from the block amax.  Reading: t = (amax_b / 6) * s_enc,
 * each operation rounded to fp32, then E4M3 round-to-nearest-even with
 * saturation.
 */
uint8_t orc_block_scale(float amax_b, float s_enc)
{
    float t = (amax_b / 6.0f) * s_enc;
    return orc_e4m3_encode_rne_sat(t);
}

/*
 * Per-element factor that maps x into E2M1 range: f = s_enc / S_b with
 * S_b the decoded block scale, or 0 if S_b is 0 (the whole block becomes
 * signed zeros).  A quotient that overflows is clamped to FLT_MAX, so that
 * zero elements stay zero (0 * f, never 0 * inf) and nonzero ones saturate.
 */
float orc_block_factor(uint8_t sb, float s_enc)
{
    float S = orc_e4m3_decode(sb);
    if (!(S > 0.0f)) return 0.0f;
    float f = s_enc / S;
    return (f > FLT_MAX) ? FLT_MAX : f;
}

static void put_code(uint8_t* row, int64_t col, uint8_t code)
{
    uint8_t* p = row + (col >> 1);
    if (col & 1) *p = (uint8_t)((*p & 0x0F) | (code << 4));
    else *p = (uint8_t)((*p & 0xF0) | code);
}

/* ------------------------------------------------------------------------ */
/* Quantisers.                                                              */
/* ------------------------------------------------------------------------ */

/*
 * NVFP4 quantisation of a row-major bf16 matrix (rows x cols).
 *   block = 1x16 : one E4M3 scale per 16 consecutive elements of a row
 *                  ([P1] TZ 2.A: 16 elements per block);
 *                  scales laid out rows x cols/16.
 *   block = 16x16: one scale per 16x16 tile ([P1] TZ 2.B.3, for weights, so
 *                  that the forward and backward passes see the same values);
 *                  scales laid out rows/16 x cols/16.
 *   rounding      : RNE or SR ([P1] TZ 2.B.4).
 * codes: rows x cols/2 bytes, element (r, c) in byte r*cols/2 + c/2, even c
 * in the low nibble.  amax_in, if not NULL, replaces the computed amax.
 * idx0 is added to every SR draw index (r*cols + c): a slice of rows of a
 * larger tensor, quantised with that tensor's amax and idx0 = its first row
 * times cols, gets exactly the codes of those rows in the whole tensor.
 */
int orc_quantize(const uint16_t* x, int64_t rows, int64_t cols, int block, int rounding,
                 uint64_t seed, uint64_t idx0, const float* amax_in, uint8_t* codes,
                 uint8_t* scales, float* amax_out, float* s_enc_out)
{
    if (rows < 0 || cols < 0 || cols % 16 != 0) return ORC_ERR_SHAPE;
    if (block == ORC_BLOCK_16X16 && rows % 16 != 0) return ORC_ERR_SHAPE;
    if (block != ORC_BLOCK_1X16 && block != ORC_BLOCK_16X16) return ORC_ERR_MODE;
    if (rounding != ORC_RNE && rounding != ORC_SR) return ORC_ERR_MODE;

    /* step 1: tensor amax */
    float amax = 0.0f;
    if (amax_in) {
        amax = *amax_in;
    } else {
        for (int64_t i = 0; i < rows * cols; ++i) {
            float a = fabsf(bf16_to_f32(x[i]));
            if (a > amax) amax = a;
        }
    }
    /* step 2: tensor scale */
    float s_enc = orc_tensor_scale(amax);
    *amax_out = amax;
    *s_enc_out = s_enc;

    int64_t nb = cols / 16;
    /* step 3: block scales */
    if (block == ORC_BLOCK_1X16) {
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t b = 0; b < nb; ++b) {
                float am = 0.0f;
                for (int i = 0; i < 16; ++i) {
                    float a = fabsf(bf16_to_f32(x[r * cols + 16 * b + i]));
                    if (a > am) am = a;
                }
                scales[r * nb + b] = orc_block_scale(am, s_enc);
            }
    } else {
#pragma omp parallel for schedule(static)
        for (int64_t tr = 0; tr < rows / 16; ++tr)
            for (int64_t b = 0; b < nb; ++b) {
                float am = 0.0f;
                for (int i = 0; i < 16; ++i)
                    for (int j = 0; j < 16; ++j) {
                        float a = fabsf(bf16_to_f32(x[(16 * tr + i) * cols + 16 * b + j]));
                        if (a > am) am = a;
                    }
                scales[tr * nb + b] = orc_block_scale(am, s_enc);
            }
    }

    /* step 4: element codes */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        uint8_t* crow = codes + r * (cols / 2);
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t sb = (block == ORC_BLOCK_1X16) ? scales[r * nb + c / 16]
                                                   : scales[(r / 16) * nb + c / 16];
            float f = orc_block_factor(sb, s_enc);
            float y = bf16_to_f32(x[r * cols + c]) * f;
            uint8_t code = (rounding == ORC_RNE)
                               ? orc_e2m1_encode_rne(y)
                               : orc_e2m1_encode_sr(y, orc_sr_draw(seed, idx0 + (uint64_t)(r * cols + c)));
            put_code(crow, c, code);
        }
    }
    return ORC_OK;
}

/*
 * 16-point random Hadamard transform of one vector ([P1] TZ 2.B.2: a 16x16
 * Hadamard rotation spreads outliers before quantisation).  Reading:
 * v <- (1/4) * H16 * D * v with H16 the Sylvester Hadamard matrix
 * (H[i][k] = (-1)^popcount(i & k)) and D = diag(d), d_i = -1 iff bit i of
 * sign_mask is set.  Because the codes are fp32 decisions, the rounding order
 * is part of the definition: signs first, then the radix-2 butterfly with
 * strides 1, 2, 4, 8, each sum and difference rounded to fp32, then the exact
 * multiplication by 1/4.
 */
void orc_rht16(const float* in, uint32_t sign_mask, float* out)
{
    float v[16];
    for (int i = 0; i < 16; ++i) v[i] = ((sign_mask >> i) & 1) ? -in[i] : in[i];
    for (int h = 1; h < 16; h <<= 1)
        for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    for (int i = 0; i < 16; ++i) out[i] = v[i] * 0.25f;
}

/*
 * Transformed, transposed wgrad operand in fp32 (no quantisation):
 * out[c * tokens + 16*j + i] = RHT of (x[16j+0..15, c])[i].
 * x is tokens x channels, row-major with leading dimension channels.
 */
int orc_rht_transform(const uint16_t* x, int64_t tokens, int64_t channels, uint32_t sign_mask,
                      float* out)
{
    if (tokens < 0 || channels < 0 || tokens % 16 != 0) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < channels; ++c)
        for (int64_t j = 0; j < tokens / 16; ++j) {
            float v[16];
            for (int i = 0; i < 16; ++i) v[i] = bf16_to_f32(x[(16 * j + i) * channels + c]);
            orc_rht16(v, sign_mask, out + c * tokens + 16 * j);
        }
    return ORC_OK;
}

/*
 * Wgrad operand: RHT along the token dimension, transpose to
 * channels x tokens, then 1x16 NVFP4 quantisation whose blocks are the
 * 16-token chunks of the transform ([P1] TZ 2.B.2: RHT only on the inputs of
 * the weight-gradient GEMM).  The tensor amax is taken over the transformed
 * values (reading).  SR draws use the index c*tokens + t of the transposed
 * layout.  codes: channels x tokens/2; scales: channels x tokens/16.
 * idx0 is added to every SR draw index, as in orc_quantize (for a slice of
 * channels: its first channel times tokens).
 */
int orc_rht_quantize(const uint16_t* x, int64_t tokens, int64_t channels, uint32_t sign_mask,
                     int rounding, uint64_t seed, uint64_t idx0, const float* amax_in,
                     uint8_t* codes, uint8_t* scales, float* amax_out, float* s_enc_out)
{
    if (tokens < 0 || channels < 0 || tokens % 16 != 0) return ORC_ERR_SHAPE;
    if (rounding != ORC_RNE && rounding != ORC_SR) return ORC_ERR_MODE;
    int64_t nb = tokens / 16;

    /* step 1: amax of the transformed operand */
    float amax = 0.0f;
    if (amax_in) {
        amax = *amax_in;
    } else {
        for (int64_t c = 0; c < channels; ++c)
            for (int64_t j = 0; j < nb; ++j) {
                float v[16], w[16];
                for (int i = 0; i < 16; ++i) v[i] = bf16_to_f32(x[(16 * j + i) * channels + c]);
                orc_rht16(v, sign_mask, w);
                for (int i = 0; i < 16; ++i)
                    if (fabsf(w[i]) > amax) amax = fabsf(w[i]);
            }
    }
    float s_enc = orc_tensor_scale(amax);
    *amax_out = amax;
    *s_enc_out = s_enc;

    /* steps 2-4 per (channel, chunk): block scale, factor, codes */
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < channels; ++c)
        for (int64_t j = 0; j < nb; ++j) {
            float v[16], w[16];
            for (int i = 0; i < 16; ++i) v[i] = bf16_to_f32(x[(16 * j + i) * channels + c]);
            orc_rht16(v, sign_mask, w);
            float am = 0.0f;
            for (int i = 0; i < 16; ++i)
                if (fabsf(w[i]) > am) am = fabsf(w[i]);
            uint8_t sb = orc_block_scale(am, s_enc);
            scales[c * nb + j] = sb;
            float f = orc_block_factor(sb, s_enc);
            for (int i = 0; i < 16; ++i) {
                float y = w[i] * f;
                int64_t t = 16 * j + i;
                uint8_t code = (rounding == ORC_RNE)
                                   ? orc_e2m1_encode_rne(y)
                                   : orc_e2m1_encode_sr(y, orc_sr_draw(seed, idx0 + (uint64_t)(c * tokens + t)));
                put_code(codes + c * (tokens / 2), t, code);
            }
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* RHT sizes other than 16 (ablation; [P1] TZ 2.B.2 reports 16 x 16 as the  */
/* best size for large models, so others were compared).                    */
/* ------------------------------------------------------------------------ */

/*
 * Reading: the D-point transform generalises the 16-point one unchanged in
 * form -- v <- 2^-(log2 D / 2) * H_D * diag(d) * v, signs first, then the
 * radix-2 butterfly with strides 1, 2, ..., D/2 (each sum and difference
 * rounded to fp32), then the exact power-of-two normalisation -- for the
 * sizes whose normalisation 1/sqrt(D) is a power of two: D = 4, 16, 64.
 * d_i = -1 iff bit i of the 64-bit sign word is set; the 64 signs are
 * words 0 (bits 0-31) and 1 (bits 32-63) of the Philox block that gives the
 * 16-point signs, so the first 16 agree with orc_rht_sign_mask.
 */
uint64_t orc_rht_signs64(uint64_t seed)
{
    uint32_t ctr[4] = {0u, 0u, 0u, 1u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    return (uint64_t)w[0] | ((uint64_t)w[1] << 32);
}

void orc_rht_sized(const float* in, int D, uint64_t signs, float* out)
{
    float v[64];
    for (int i = 0; i < D; ++i) v[i] = ((signs >> i) & 1) ? -in[i] : in[i];
    for (int h = 1; h < D; h <<= 1)
        for (int i = 0; i < D; ++i)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    const float norm = D == 1 ? 1.0f : (D == 4 ? 0.5f : (D == 16 ? 0.25f : 0.125f));
    for (int i = 0; i < D; ++i) out[i] = v[i] * norm;
}

/* D = 1 is no transform (only the sign of bit 0): the plain transposing
   quantiser, the baseline of the size comparison */
static int rht_size_ok(int D) { return D == 1 || D == 4 || D == 16 || D == 64; }

/*
 * The wgrad operand with a D-point transform along tokens (D = 4, 16, 64),
 * then transpose and 1x16 quantisation exactly as orc_rht_quantize (blocks
 * of 16 tokens, amax over the transformed tensor, SR index c*tokens + t).
 * tokens must be a multiple of 16 and of D.
 */
int orc_rht_quantize_sized(const uint16_t* x, int64_t tokens, int64_t channels, int D,
                           uint64_t signs, int rounding, uint64_t seed, const float* amax_in,
                           uint8_t* codes, uint8_t* scales, float* amax_out, float* s_enc_out)
{
    if (!rht_size_ok(D)) return ORC_ERR_MODE;
    if (rounding != ORC_RNE && rounding != ORC_SR) return ORC_ERR_MODE;
    if (tokens < 0 || channels < 0 || tokens % 16 != 0 || tokens % D != 0) return ORC_ERR_SHAPE;
    const int64_t nb = tokens / 16;

    /* step 1: amax of the transformed operand */
    float amax = 0.0f;
    if (amax_in) {
        amax = *amax_in;
    } else {
        for (int64_t c = 0; c < channels; ++c)
            for (int64_t j = 0; j < tokens / D; ++j) {
                float v[64], w[64];
                for (int i = 0; i < D; ++i) v[i] = bf16_to_f32(x[(D * j + i) * channels + c]);
                orc_rht_sized(v, D, signs, w);
                for (int i = 0; i < D; ++i)
                    if (fabsf(w[i]) > amax) amax = fabsf(w[i]);
            }
    }
    const float s_enc = orc_tensor_scale(amax);
    *amax_out = amax;
    *s_enc_out = s_enc;

    /* steps 2-4 per (channel, 16-token block): the transformed values of
       the block (from the D-token chunk that holds it, or from its 16 / D
       chunks when D = 4), block scale, factor, codes */
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < channels; ++c)
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t t0 = 16 * b;
            const int64_t u0 = D >= 16 ? (t0 / D) * D : t0;   /* first transformed chunk */
            const int64_t u1 = D >= 16 ? u0 + D : t0 + 16;      /* end of the last one */
            float w16[16];
            for (int64_t u = u0; u < u1; u += D) {
                float v[64], w[64];
                for (int i = 0; i < D; ++i) v[i] = bf16_to_f32(x[(u + i) * channels + c]);
                orc_rht_sized(v, D, signs, w);
                for (int i = 0; i < D; ++i)
                    if (u + i >= t0 && u + i < t0 + 16) w16[u + i - t0] = w[i];
            }
            float am = 0.0f;
            for (int i = 0; i < 16; ++i)
                if (fabsf(w16[i]) > am) am = fabsf(w16[i]);
            const uint8_t sb = orc_block_scale(am, s_enc);
            scales[c * nb + b] = sb;
            const float f = orc_block_factor(sb, s_enc);
            for (int i = 0; i < 16; ++i) {
                const float y = w16[i] * f;
                const int64_t t = t0 + i;
                const uint8_t code = (rounding == ORC_RNE)
                                         ? orc_e2m1_encode_rne(y)
                                         : orc_e2m1_encode_sr(y, orc_sr_draw(seed, (uint64_t)(c * tokens + t)));
                put_code(codes + c * (tokens / 2), t, code);
            }
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* RHT on the fprop / dgrad operands (ablation; [P1] TZ 2.B.2 reports no    */
/* significant benefit there, which is why the recipe keeps it to wgrad).   */
/* ------------------------------------------------------------------------ */

/*
 * Reading: for fprop and dgrad the transform runs along the contraction
 * dimension, i.e. along the rows of X, W (fprop) and dY, W^T (dgrad): the
 * 16-point transform of R-11 on every aligned 16-element chunk of a row --
 * exactly the chunk of a 1x16 block, and a row of a 16x16 tile -- with one
 * sign vector for both operands of a GEMM, so that (A Q^T)(B Q^T)^T = A B^T.
 * Then NVFP4 quantisation as orc_quantize (tensor amax over the transformed
 * values; 1x16 or 16x16 blocks; SR index r * cols + c).
 */
int orc_quantize_rht_rows(const uint16_t* x, int64_t rows, int64_t cols, int block,
                          uint32_t sign_mask, int rounding, uint64_t seed, const float* amax_in,
                          uint8_t* codes, uint8_t* scales, float* amax_out, float* s_enc_out)
{
    if (rows < 0 || cols < 0 || cols % 16 != 0) return ORC_ERR_SHAPE;
    if (block == ORC_BLOCK_16X16 && rows % 16 != 0) return ORC_ERR_SHAPE;
    if (block != ORC_BLOCK_1X16 && block != ORC_BLOCK_16X16) return ORC_ERR_MODE;
    if (rounding != ORC_RNE && rounding != ORC_SR) return ORC_ERR_MODE;
    const int64_t nb = cols / 16;

    /* the transformed rows (fp32), chunk by chunk */
    float* t = (float*)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
    if (!t) return ORC_ERR_SHAPE;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float v[16];
            for (int i = 0; i < 16; ++i) v[i] = bf16_to_f32(x[r * cols + 16 * b + i]);
            orc_rht16(v, sign_mask, t + r * cols + 16 * b);
        }

    /* step 1: tensor amax over the transformed values */
    float amax = 0.0f;
    if (amax_in) {
        amax = *amax_in;
    } else {
        for (int64_t i = 0; i < rows * cols; ++i)
            if (fabsf(t[i]) > amax) amax = fabsf(t[i]);
    }
    const float s_enc = orc_tensor_scale(amax);
    *amax_out = amax;
    *s_enc_out = s_enc;

    /* step 2: block scales */
    if (block == ORC_BLOCK_1X16) {
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t b = 0; b < nb; ++b) {
                float am = 0.0f;
                for (int i = 0; i < 16; ++i)
                    if (fabsf(t[r * cols + 16 * b + i]) > am) am = fabsf(t[r * cols + 16 * b + i]);
                scales[r * nb + b] = orc_block_scale(am, s_enc);
            }
    } else {
#pragma omp parallel for schedule(static)
        for (int64_t tr = 0; tr < rows / 16; ++tr)
            for (int64_t b = 0; b < nb; ++b) {
                float am = 0.0f;
                for (int i = 0; i < 16; ++i)
                    for (int j = 0; j < 16; ++j)
                        if (fabsf(t[(16 * tr + i) * cols + 16 * b + j]) > am)
                            am = fabsf(t[(16 * tr + i) * cols + 16 * b + j]);
                scales[tr * nb + b] = orc_block_scale(am, s_enc);
            }
    }

    /* step 3: element codes */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            const uint8_t sb = block == ORC_BLOCK_1X16 ? scales[r * nb + c / 16]
                                                       : scales[(r / 16) * nb + c / 16];
            const float y = t[r * cols + c] * orc_block_factor(sb, s_enc);
            const uint8_t code = (rounding == ORC_RNE)
                                     ? orc_e2m1_encode_rne(y)
                                     : orc_e2m1_encode_sr(y, orc_sr_draw(seed, (uint64_t)(r * cols + c)));
            put_code(codes + r * (cols / 2), c, code);
        }
    free(t);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* MXFP4, the format NVFP4 is compared with ([P1] TZ 2.A).                  */
/* ------------------------------------------------------------------------ */

/*
 * [P1] TZ 2.A sets NVFP4 against MXFP4: E2M1 elements in blocks of 32 that
 * share a power-of-two scale stored as UE8M0, with no tensor-level scale.
 * The pages stop there.  Reading (the OCP Microscaling Formats
 * specification, v1.0, which defines MXFP4): the shared exponent of a block
 * is floor(log2(amax_b)) - 2, where 2 is the exponent of E2M1's largest
 * value 6 = 1.5 * 2^2, clamped to the UE8M0 range [-127, 127]; an all-zero
 * block takes -127.  The scale byte is the exponent + 127.  Inputs are
 * finite.
 */
int orc_mx_exponent(float amax_b)
{
    if (!(amax_b > 0.0f)) return -127;
    int ex;
    (void)frexpf(amax_b, &ex);  /* amax_b = m * 2^ex, m in [0.5, 1) */
    int e = (ex - 1) - 2;       /* floor(log2(amax_b)) - 2 */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/*
 * The 32 values of MX block b of output row r (fp32), for the three
 * layouts of orc_mx_quantize.
 */
static void mx_block_values(const uint16_t* x, int64_t rows, int64_t cols, int mode,
                            uint32_t sign_mask, int64_t r, int64_t b, float* v)
{
    if (mode == 0) {
        for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(x[r * cols + 32 * b + i]);
        return;
    }
    /* modes 1, 2: output row r is input column r; block b is input rows 32b.. */
    for (int i = 0; i < 32; ++i) v[i] = bf16_to_f32(x[(32 * b + i) * cols + r]);
    if (mode == 2) {
        float w[16];
        for (int h = 0; h < 2; ++h) {
            orc_rht16(v + 16 * h, sign_mask, w);
            for (int i = 0; i < 16; ++i) v[16 * h + i] = w[i];
        }
    }
    (void)rows;
}

/*
 * MXFP4 quantisation of a row-major bf16 matrix x (rows x cols).
 *   mode 0: blocks of 32 along each row; output rows x cols.
 *   mode 1: the transposed matrix, blocks of 32 along each column of x;
 *           output cols x rows.
 *   mode 2: as mode 1 after the 16-point random Hadamard transform of every
 *           aligned 16-row chunk of each column (orc_rht16, sign_mask) --
 *           the wgrad operand of the recipe, [P1] TZ 2.B.2.
 * Each element: y = v * 2^-e (fp32; exact unless it underflows, where every
 * rounding gives a zero of the same sign), coded onto the E2M1 grid by RNE
 * (saturating) or by SR with the draw of its index r * out_cols + c in the
 * output layout ([P1] TZ 2.B.4), exactly as for NVFP4.
 * codes: out_rows x out_cols/2; scales: out_rows x out_cols/32 (UE8M0).
 */
int orc_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int mode, uint32_t sign_mask,
                    int rounding, uint64_t seed, uint8_t* codes, uint8_t* scales)
{
    if (rows < 0 || cols < 0) return ORC_ERR_SHAPE;
    if (mode < 0 || mode > 2) return ORC_ERR_MODE;
    if (rounding != ORC_RNE && rounding != ORC_SR) return ORC_ERR_MODE;
    if (mode == 0 && cols % 32 != 0) return ORC_ERR_SHAPE;
    if (mode != 0 && rows % 32 != 0) return ORC_ERR_SHAPE;
    const int64_t out_rows = mode == 0 ? rows : cols;
    const int64_t out_cols = mode == 0 ? cols : rows;
    const int64_t nb = out_cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < out_rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            float v[32];
            mx_block_values(x, rows, cols, mode, sign_mask, r, b, v);
            float am = 0.0f;
            for (int i = 0; i < 32; ++i)
                if (fabsf(v[i]) > am) am = fabsf(v[i]);
            const int e = orc_mx_exponent(am);
            scales[r * nb + b] = (uint8_t)(e + 127);
            const float f = ldexpf(1.0f, -e);
            for (int i = 0; i < 32; ++i) {
                const float y = v[i] * f;
                const int64_t c = 32 * b + i;
                const uint8_t code = (rounding == ORC_RNE)
                                         ? orc_e2m1_encode_rne(y)
                                         : orc_e2m1_encode_sr(y, orc_sr_draw(seed, (uint64_t)(r * out_cols + c)));
                put_code(codes + r * (out_cols / 2), c, code);
            }
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Diagnostic GEMM with fp32 accumulation.                                  */
/* ------------------------------------------------------------------------ */

/*
 * C[m, n] = alpha * sum_k A^[m, k] * B^[n, k] over dequantised NVFP4
 * operands, both stored rows x K with 16-element blocks along K.  Each
 * 16-block partial is exact (integer sum of products of doubled E2M1 values,
 * times two E4M3 scales); the partials are added in fp32 in block order and
 * the sum is multiplied by alpha = (1/s_enc_A) * (1/s_enc_B), the product of
 * the two FP32 tensor decode scales ("Pretraining Large Language Models with
 * NVFP4", Technische Zusammenfassung 2.A: one FP32 scale per tensor).  That
 * product is formed in fp32 while it is a normal number; below fp32's normal
 * range (tiny tensor maxima) its significand (the rounded product of the two
 * factors' significands) and its exponent are kept apart, and the output is
 * ldexp(RN(acc * significand), exponent) -- the value of RN(acc * alpha)
 * with alpha held to 24 significant bits instead of a subnormal.  The reference
 * GEMM used by the parity tests is the fp64 product of the dequantised
 * matrices; this fp32 variant only bounds how far an fp32-accumulating GEMM
 * may sit from it.
 *   a_scale_rows_per: 1 for 1x16 operands, 16 for 16x16 operands (same for b).
 */
int orc_gemm_fp32(const uint8_t* a_codes, const uint8_t* a_scales, int a_scale_rows_per,
                  float a_s_enc, const uint8_t* b_codes, const uint8_t* b_scales,
                  int b_scale_rows_per, float b_s_enc, int64_t M, int64_t N, int64_t K,
                  float* c)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return ORC_ERR_SHAPE;
    int64_t nb = K / 16;
    float da = 1.0f / a_s_enc, db = 1.0f / b_s_enc;
    float alpha = da * db;
    int alpha_exp = 0;
    if (!(alpha >= FLT_MIN)) {
        int ea, eb;
        float ma = frexpf(da, &ea), mb = frexpf(db, &eb);
        alpha = ma * mb;
        alpha_exp = ea + eb;
    }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t b = 0; b < nb; ++b) {
                int32_t P = 0;
                for (int i = 0; i < 16; ++i) {
                    int64_t k = 16 * b + i;
                    uint8_t ca = (uint8_t)((a_codes[m * (K / 2) + k / 2] >> (4 * (k & 1))) & 15);
                    uint8_t cb = (uint8_t)((b_codes[n * (K / 2) + k / 2] >> (4 * (k & 1))) & 15);
                    P += (int32_t)(2.0 * orc_e2m1_decode(ca)) * (int32_t)(2.0 * orc_e2m1_decode(cb));
                }
                float SA = orc_e4m3_decode(a_scales[(m / a_scale_rows_per) * nb + b]);
                float SB = orc_e4m3_decode(b_scales[(n / b_scale_rows_per) * nb + b]);
                float term = ((float)P * 0.25f * SA) * SB;
                acc += term;
            }
            float out = acc * alpha;
            c[m * N + n] = alpha_exp ? ldexpf(out, alpha_exp) : out;
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Array forms of the scalar steps, for the tests.                          */
/* ------------------------------------------------------------------------ */

void orc_e2m1_encode_rne_n(const float* y, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_encode_rne(y[i]);
}

void orc_e2m1_encode_sr_n(const float* y, const uint16_t* u, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_encode_sr(y[i], u[i]);
}

void orc_e4m3_encode_n(const float* t, int64_t n, uint8_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode_rne_sat(t[i]);
}

void orc_sr_draw_n(uint64_t seed, uint64_t idx0, int64_t n, uint16_t* out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_sr_draw(seed, idx0 + (uint64_t)i);
}
