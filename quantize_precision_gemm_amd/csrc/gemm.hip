// gemm.hip -- GEMMs on gfx950 matrix cores: over NVFP4 operands, and over
// bf16 operands for the layers that stay in high precision.
//
// Passes: "Pretraining Large Language Models with NVFP4" (gist.science
// summary), Technische Zusammenfassung 2.B.2 (Fprop, Dgrad, Wgrad GEMMs of a
// linear layer); format 2.A (E2M1 codes, E4M3 scale per 16 elements, FP32
// tensor scale); 2.B.1 (a few layers keep BF16).
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
// The kernel computes C[m, n] = alpha sum_k A[m, k] B[n, k].  NVFP4 operands
// are always "rows x K" with K contiguous (the dgrad weight operand is the
// transposed 16x16-block copy written by the quantiser).  A bf16 operand is
// either "rows x K" (layout N) or "K x rows" (layout T, rows contiguous), so
// the three bf16 passes read X, W and dY where they lie.
//
// A workgroup of 8 waves (two per SIMD) computes a 256x256 tile in K steps
// of 64.  Per step threads 0-255 bring the A tile and threads 256-511 the B
// tile into a 16-bit LDS stage (256 rows of 64 values): an NVFP4 thread
// decodes one row's 32 code bytes and 4 scales, so each element is decoded
// once per workgroup; a bf16 thread moves 8 16-byte pieces, transposing an
// 8x8 block in registers for layout T.  Each wave then runs 4x2 MFMA
// 32x32x16 tiles (a 128x64 slab, 128 fp32 accumulators) over the stage.  Two
// LDS stages alternate: while the MFMAs consume one, the next step's data
// (loaded from global memory earlier) is written into the other.  NVFP4 rows
// are small (9 registers), so three register stages keep their global loads
// three steps ahead of the MFMAs; bf16 rows (32 registers) get one stage and
// load one step ahead.  Two waves per SIMD
// let one wave's MFMAs cover the other's waits.  The epilogue stages 32
// output rows per wave through LDS and stores 16-byte row segments.
//
// Lane layout of v_mfma_f32_32x32x16_{f16,bf16}: lane l supplies row (A) or
// column (B) l % 32 and the 8 consecutive k 8*(l/32) .. +7 of the 16-wide
// step; accumulator j of lane l is row (j/4)*8 + (l/32)*4 + j%4, column l % 32.
#include <utility>

#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kBM = 256, kBN = 256, kKS = 64;  // workgroup tile and K step
constexpr int kRowBytes = 144;                 // LDS row: 64 16-bit values (128 B) + 16 B pad
constexpr int kOpBytes = 256 * kRowBytes;      // one operand, one stage

// Kernel arguments of one operand; fields a source does not use stay zero.
struct OpArgs {
    const void* data;       // NVFP4 codes, or bf16 values
    int64_t ld;             // bytes (codes) or elements (bf16) between consecutive rows in memory
    const uint8_t* scales;  // NVFP4: E4M3 block scales
    int64_t ld_scales;
    int scale_shift;        // NVFP4: scale row = row >> scale_shift
    const float* s_enc;     // NVFP4: tensor encode scale
    int trans;              // bf16: 1 = stored K x rows (layout T), 0 = rows x K (layout N)
};

// --- NVFP4 operand: one thread per tile row --------------------------------

struct Nvfp4Src {
    struct Row {  // one row's K step: 32 code bytes (64 k) and 4 scale bytes
        uint4 c0, c1;
        uint32_t s;
    };
    typedef half8_t frag_t;
    static constexpr bool kDeep = true;  // rows are small: three register stages
    const uint8_t* codes;
    const uint8_t* scales;
    int64_t nblk;
    int rid;

    // rid: this thread's row within the tile, r0: the tile's first row,
    // lim: rows of the operand (rows past it re-read the last row; they are
    // never stored)
    __device__ __forceinline__ Nvfp4Src(const OpArgs& o, int rid_, int64_t r0, int64_t lim,
                                        int64_t K)
    {
        rid = rid_;
        int64_t r = r0 + rid;
        r = r < lim ? r : lim - 1;
        codes = static_cast<const uint8_t*>(o.data) + r * o.ld;
        scales = o.scales + (r >> o.scale_shift) * o.ld_scales;
        nblk = K >> 4;
    }
    __device__ __forceinline__ void load_full(int64_t k0, Row& w) const
    {
        const uint4* p = reinterpret_cast<const uint4*>(codes + (k0 >> 1));
        w.c0 = p[0];
        w.c1 = p[1];
        w.s = *reinterpret_cast<const uint32_t*>(scales + (k0 >> 4));
    }
    // partial last step: missing blocks get zero codes and zero scales
    __device__ __forceinline__ void load_tail(int64_t k0, Row& w) const
    {
        const int64_t b0 = k0 >> 4;
        const uint4* p = reinterpret_cast<const uint4*>(codes + (k0 >> 1));
        w.c0 = (b0 < nblk) ? p[0] : make_uint4(0, 0, 0, 0);
        w.c1 = (b0 + 2 < nblk) ? p[1] : make_uint4(0, 0, 0, 0);
        w.s = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (b0 + j < nblk) w.s |= (uint32_t)scales[b0 + j] << (8 * j);
    }
    // decode 64 codes (4 blocks) to exact fp16 q * S into the row's 128 LDS bytes
    __device__ __forceinline__ void store(const Row& w, uint8_t* __restrict__ op) const
    {
        uint8_t* dst = op + rid * kRowBytes;
        const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.s, 1.0f, false);
        const half2_t sb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.s, 1.0f, true);
        const half2_t ss[4] = {__builtin_shufflevector(sa, sa, 0, 0), __builtin_shufflevector(sa, sa, 1, 1),
                               __builtin_shufflevector(sb, sb, 0, 0), __builtin_shufflevector(sb, sb, 1, 1)};
        const uint32_t c[8] = {w.c0.x, w.c0.y, w.c0.z, w.c0.w, w.c1.x, w.c1.y, w.c1.z, w.c1.w};
#pragma unroll
        for (int d = 0; d < 8; ++d) {  // dword d: elements 8d .. 8d+7, block d / 2
            const half2_t S = ss[d >> 1];
            half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 0) * S;
            half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 1) * S;
            half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 2) * S;
            half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c[d], 1.0f, 3) * S;
            uint4 v;
            v.x = __builtin_bit_cast(uint32_t, p0);
            v.y = __builtin_bit_cast(uint32_t, p1);
            v.z = __builtin_bit_cast(uint32_t, p2);
            v.w = __builtin_bit_cast(uint32_t, p3);
            *reinterpret_cast<uint4*>(dst + 16 * d) = v;
        }
    }
    __device__ __forceinline__ static float16_t mfma(const frag_t& a, const frag_t& b, const float16_t& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// --- bf16 operand ----------------------------------------------------------
//
// Thread rid moves 8 pieces of 16 bytes (8 values) per step; kg = rid % 8
// names the 8-wide k group of the step it covers and c = rid / 8 the rows.
// Layout N (rows x K): piece j is row c + 32 j, k group kg -- a wave's load
//   covers 8 full 128-byte row segments.
// Layout T (K x rows): piece j is k row 8 kg + j, rows 8c .. 8c+7 -- again 8
//   full 128-byte segments per wave load; the 8x8 block is transposed in
//   registers so that piece i becomes row 8c + i, k group kg.
// Either way the 8 lanes of equal c write 128 consecutive LDS bytes, which
// keeps the stage writes free of bank conflicts.  K and the row count are
// multiples of 8, so a piece is wholly inside or wholly outside the operand.
// kMode: 0 = both operands N, 1 = both T, 2 = per operand (OpArgs::trans);
// in mode 2 both layouts' arithmetic runs and a select keeps one, so the two
// halves of the workgroup run the same instructions.
template <int kMode>
struct Bf16Src {
    struct Row {
        uint4 v[8];
    };
    typedef bf16x8_t frag_t;
    static constexpr bool kDeep = false;  // 32 registers per stage: one stage
    const uint16_t* base;  // piece 0 of step 0
    int64_t ld, K, kstride, jstride;
    int kg, c, cmax;
    bool t_;

    __device__ __forceinline__ bool trans() const { return kMode == 2 ? t_ : kMode == 1; }

    __device__ __forceinline__ Bf16Src(const OpArgs& o, int rid, int64_t r0, int64_t lim, int64_t K_)
    {
        t_ = o.trans != 0;
        ld = o.ld;
        K = K_;
        kg = rid & 7;
        c = rid >> 3;
        const uint16_t* d = static_cast<const uint16_t*>(o.data);
        if (trans()) {
            int64_t rc = r0 + 8 * c;  // first row of the piece; past the end: re-read the last piece
            rc = rc + 8 <= lim ? rc : lim - 8;
            base = d + (int64_t)(8 * kg) * ld + rc;
            cmax = 0x7fffffff;
            kstride = ld;
            jstride = ld;
        } else {
            base = d + r0 * ld + 8 * kg;
            const int64_t left = lim - r0 - 1;  // last valid row offset within the tile
            cmax = left < 255 ? (int)left : 255;
            kstride = 1;
            jstride = ld;
        }
    }
    // row offset (N: row c + 32 j clamped; T: k row j) times ld
    __device__ __forceinline__ const uint4* piece(int64_t k0, int j) const
    {
        const int r = trans() ? j : min(c + 32 * j, cmax);
        return reinterpret_cast<const uint4*>(base + (int64_t)r * jstride + k0 * kstride);
    }
    __device__ __forceinline__ void load_full(int64_t k0, Row& w) const
    {
#pragma unroll
        for (int j = 0; j < 8; ++j) w.v[j] = *piece(k0, j);
    }
    // partial last step: pieces past K read as zero
    __device__ __forceinline__ void load_tail(int64_t k0, Row& w) const
    {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t k = k0 + 8 * kg + (trans() ? j : 0);
            w.v[j] = (k < K) ? *piece(k0, j) : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void store(const Row& w, uint8_t* __restrict__ op) const
    {
        // T: w.v[j] holds rows 8c .. 8c+7 at k = 8kg + j, two rows per dword;
        // row 2d + h of the block takes half h of dword d of every piece
        const uint32_t* v = reinterpret_cast<const uint32_t*>(w.v);
        const int rbase = trans() ? 8 * c : c, rstep = trans() ? 1 : 32;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int d = i >> 1;
            const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
            uint4 t = w.v[i];
            if (kMode != 0) {
                uint4 u;
                u.x = __builtin_amdgcn_perm(v[4 * 1 + d], v[4 * 0 + d], sel);
                u.y = __builtin_amdgcn_perm(v[4 * 3 + d], v[4 * 2 + d], sel);
                u.z = __builtin_amdgcn_perm(v[4 * 5 + d], v[4 * 4 + d], sel);
                u.w = __builtin_amdgcn_perm(v[4 * 7 + d], v[4 * 6 + d], sel);
                if (trans()) t = u;
            }
            *reinterpret_cast<uint4*>(op + (rbase + rstep * i) * kRowBytes + 16 * kg) = t;
        }
    }
    __device__ __forceinline__ static float16_t mfma(const frag_t& a, const frag_t& b, const float16_t& c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Instruction-schedule hint for one K step (32 MFMAs per wave): the first
// half of the MFMAs is interleaved with the LDS fragment reads only; the
// second half also carries the next step's LDS writes and the VALU work
// feeding them (the NVFP4 decode, the bf16 transpose), which gives the
// global loads behind them as much time as possible to land.
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

template <class Src, bool kOutF32>
__global__ __launch_bounds__(512, 1) void k_gemm_nt(OpArgs A, OpArgs B, int64_t M, int64_t N,
                                                    int64_t K, void* __restrict__ c, int64_t ldc)
{
    typedef typename Src::Row Row;
    typedef typename Src::frag_t frag_t;
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

    // threads 0..255 bring the A tile into LDS, 256..511 the B tile
    const bool is_b = tid >= 256;
    const int rid = tid & 255;
    const Src src(is_b ? B : A, rid, is_b ? tile_n * kBN : tile_m * kBM, is_b ? N : M, K);
    auto put = [&](const Row& w, int stage) { src.store(w, lds[stage][is_b ? 1 : 0]); };

    float16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int wm = wave >> 2, wn = wave & 3;
    // fragment read offsets within a stage: row (32 t + lr) of the wave's
    // 128-row A slab / 64-row B slab, k = 16 i + 8 g
    const int a_frag = (wm * 128 + lr) * kRowBytes + 16 * g;
    const int b_frag = (wn * 64 + lr) * kRowBytes + 16 * g;

    auto compute = [&](int stage) {
        const uint8_t* As = lds[stage][0];
        const uint8_t* Bs = lds[stage][1];
        frag_t af[2][4], bf[2][2];  // fragments of two sub-steps in flight
#pragma unroll
        for (int t = 0; t < 4; ++t) af[0][t] = *reinterpret_cast<const frag_t*>(As + a_frag + t * 32 * kRowBytes);
#pragma unroll
        for (int t = 0; t < 2; ++t) bf[0][t] = *reinterpret_cast<const frag_t*>(Bs + b_frag + t * 32 * kRowBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cur = i & 1, nxt = cur ^ 1;
            if (i < 3) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    af[nxt][t] = *reinterpret_cast<const frag_t*>(As + a_frag + t * 32 * kRowBytes + 32 * (i + 1));
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    bf[nxt][t] = *reinterpret_cast<const frag_t*>(Bs + b_frag + t * 32 * kRowBytes + 32 * (i + 1));
            }
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 2; ++tn) acc[tm][tn] = Src::mfma(af[cur][tm], bf[cur][tn], acc[tm][tn]);
        }
    };

    // Main loop over full K steps (the partial last step is handled after it).
    const int64_t nsteps = (K + kKS - 1) / kKS;
    const int64_t nfull = K / kKS;
    int64_t s = 0;
    Row g0, g1;
    if constexpr (Src::kDeep) {
        // global loads run three steps ahead of the MFMAs (three register
        // stages); step t's row data lives in register stage t % 3 and its
        // decoded tile in LDS stage t % 2
        Row g2;
        if (nfull > 0) {
            src.load_full(0, g0);
            // unconditional (clamped) loads keep the wait counts exact
            src.load_full((nfull > 1 ? 1 : 0) * kKS, g1);
            src.load_full((nfull > 2 ? 2 : nfull - 1) * kKS, g2);
            put(g0, 0);
        }
        __syncthreads();
        auto step = [&](auto c3, int64_t t) {
            constexpr int r = decltype(c3)::value;
            const int st = (int)(t & 1);
            Row& done = r == 0 ? g0 : (r == 1 ? g1 : g2);        // step t, already in LDS
            Row& next = r == 0 ? g1 : (r == 1 ? g2 : g0);        // step t + 1
            src.load_full((t + 3 < nfull ? t + 3 : nfull - 1) * kKS, done);
            compute(st);
            put(next, st ^ 1);  // past the last full step: harmless, never read
            interleave_step(std::make_integer_sequence<int, 32>{});
            __syncthreads();
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        for (; s + 3 <= nfull; s += 3) {
            step(I0{}, s);
            step(I1{}, s + 1);
            step(I2{}, s + 2);
        }
        if (s < nfull) step(I0{}, s++);
        if (s < nfull) step(I1{}, s++);
        if (nfull < nsteps) {  // partial last step into LDS stage nfull % 2
            src.load_tail(nfull * kKS, g0);
            put(g0, (int)(nfull & 1));
            __syncthreads();
            compute((int)(nfull & 1));
        }
    } else {
        // one register stage: the loads of step s+1 are issued before the
        // MFMAs of step s and written to LDS after them
        if (nfull > 0) {
            src.load_full(0, g0);
            put(g0, 0);
        }
        __syncthreads();
        for (; s + 2 <= nfull; s += 2) {
            src.load_full((s + 1) * kKS, g0);
            // keep the loads ahead of the MFMAs: with one register stage
            // they have only this step to land
            __builtin_amdgcn_sched_barrier(0);
            compute(0);
            put(g0, 1);
            interleave_step(std::make_integer_sequence<int, 32>{});
            __syncthreads();
            src.load_full((s + 2 < nfull ? s + 2 : nfull - 1) * kKS, g0);
            __builtin_amdgcn_sched_barrier(0);
            compute(1);
            put(g0, 0);  // harmless on the last pass: stage 0 is not read again
            interleave_step(std::make_integer_sequence<int, 32>{});
            __syncthreads();
        }
    }
    if constexpr (!Src::kDeep) {
        if (s < nfull) compute(0);  // odd number of full steps: the last one is in stage 0
        if (nfull < nsteps) {       // partial last step
            src.load_tail(nfull * kKS, g1);
            __syncthreads();
            put(g1, 1);
            __syncthreads();
            compute(1);
        }
    }

    // Epilogue: each wave stages 32 output rows at a time through LDS (fp32,
    // alpha applied) and writes them back as 16-byte row segments.
    float alpha = 1.0f;
    if (A.s_enc) alpha = (1.0f / *A.s_enc) * (1.0f / *B.s_enc);
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

template <class Src>
static void launch(const OpArgs& a, const OpArgs& b, int64_t M, int64_t N, int64_t K, void* c,
                   int64_t ldc, bool out_fp32, hipStream_t s)
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
    const dim3 grid((unsigned)tiles), block(512);
    if (out_fp32)
        hipLaunchKernelGGL((k_gemm_nt<Src, true>), grid, block, 0, s, a, b, M, N, K, c, ldc);
    else
        hipLaunchKernelGGL((k_gemm_nt<Src, false>), grid, block, 0, s, a, b, M, N, K, c, ldc);
}

void launch_gemm_nt(const GemmOperand& a, const GemmOperand& b, int64_t M, int64_t N, int64_t K,
                    void* c, int64_t ldc, bool out_fp32, hipStream_t s)
{
    const OpArgs A{a.codes, a.ld_codes, a.scales, a.ld_scales, a.scale_row_shift, a.s_enc, 0};
    const OpArgs B{b.codes, b.ld_codes, b.scales, b.ld_scales, b.scale_row_shift, b.s_enc, 0};
    launch<Nvfp4Src>(A, B, M, N, K, c, ldc, out_fp32, s);
}

void launch_bf16_gemm(const uint16_t* a, int64_t lda, bool a_t, const uint16_t* b, int64_t ldb,
                      bool b_t, int64_t M, int64_t N, int64_t K, void* c, int64_t ldc,
                      bool out_fp32, hipStream_t s)
{
    const OpArgs A{a, lda, nullptr, 0, 0, nullptr, a_t ? 1 : 0};
    const OpArgs B{b, ldb, nullptr, 0, 0, nullptr, b_t ? 1 : 0};
    if (a_t != b_t)
        launch<Bf16Src<2>>(A, B, M, N, K, c, ldc, out_fp32, s);
    else if (a_t)
        launch<Bf16Src<1>>(A, B, M, N, K, c, ldc, out_fp32, s);
    else
        launch<Bf16Src<0>>(A, B, M, N, K, c, ldc, out_fp32, s);
}

}  // namespace nvfp4
