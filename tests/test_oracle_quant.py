"""Pins of the oracle's quantisers against exact brute force and the pages' invariants.

Page: "Pretraining Large Language Models with NVFP4" (gist.science summary),
Technische Zusammenfassung:
  2.A   16-element blocks, E4M3 block scale, FP32 tensor scale; about 1/16 of
        the values of a block (its largest) are encoded at nearly FP8 precision.
  2.B.3 16x16 blocks for weights so that forward and backward passes see the
        same quantised weights.
  2.B.4 stochastic rounding for gradients (unbiased), round-to-nearest-even
        for activations and weights.
"""
import numpy as np
import pytest

import oracle
from quantize_precision_gemm_amd import workloads as wl
from tests import exact_nvfp4 as ex


def _rand_bits(rng, shape, kind):
    if kind == "normal":
        x = rng.standard_normal(shape)
    elif kind == "wide":
        x = rng.standard_normal(shape) * np.exp(rng.uniform(-30, 30, shape))
    elif kind == "tiny":
        x = rng.standard_normal(shape) * 1e-38
    elif kind == "rows":
        x = rng.standard_normal(shape) * np.exp(4 * rng.standard_normal((shape[0], 1)))
    else:
        raise ValueError(kind)
    return wl.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("kind", ["normal", "wide", "tiny", "rows"])
@pytest.mark.parametrize("rounding", [oracle.RNE, oracle.SR])
def test_brute_force_4x16(kind, rounding):
    # I-6: 4x16 inputs, every scale and code re-derived in exact arithmetic
    # (nearest over all E4M3 values, nearest over all 16 E2M1 codes).
    rng = np.random.default_rng(hash((kind, rounding)) % 2 ** 32)
    for trial in range(25):
        x = _rand_bits(rng, (4, 32), kind)
        if trial == 0:
            x[0, :5] = [0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F]  # +-0, +-min subnormal, max bf16
        seed = int(rng.integers(0, 2 ** 63))
        q = oracle.quantize(x, oracle.BLOCK_1X16, rounding, seed)
        flat = [int(v) for v in x.reshape(-1)]
        blocks = [list(range(16 * b, 16 * b + 16)) for b in range(len(flat) // 16)]
        draws = None
        if rounding == oracle.SR:
            draws = [int(v) for v in oracle.sr_draws(seed, 0, len(flat))]
        codes, sb, amax, s_enc = ex.quantize_blocks(flat, blocks, draws)
        assert np.float32(q.amax) == np.float32(float(amax))
        assert np.float32(q.s_enc) == np.float32(float(s_enc))
        assert list(q.scales.reshape(-1)) == sb
        assert list(oracle.unpack_codes(q.codes, 32).reshape(-1)) == codes


def test_brute_force_16x16_tiles():
    rng = np.random.default_rng(11)
    for trial in range(6):
        x = _rand_bits(rng, (32, 32), ["normal", "wide", "rows"][trial % 3])
        q = oracle.quantize(x, oracle.BLOCK_16X16, oracle.RNE)
        flat = [int(v) for v in x.reshape(-1)]
        blocks = []
        for tr in range(2):
            for tc in range(2):
                blocks.append([(16 * tr + i) * 32 + 16 * tc + j for i in range(16) for j in range(16)])
        codes, sb, _, _ = ex.quantize_blocks(flat, blocks)
        assert list(q.scales.reshape(-1)) == sb
        assert list(oracle.unpack_codes(q.codes, 32).reshape(-1)) == codes


def test_block_amax_element_near_fp8_precision():
    # I-4: in every block whose scale is a normal E4M3 value, the largest element
    # gets magnitude code 7 (value 6) and decodes within 2^-4 relative of its input.
    rng = np.random.default_rng(3)
    x = _rand_bits(rng, (512, 256), "rows")
    q = oracle.quantize(x, oracle.BLOCK_1X16, oracle.RNE)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    codes = oracle.unpack_codes(q.codes, 256)
    deq = oracle.dequantize(q)
    blk = np.abs(xf).reshape(512, 16, 16)
    arg = blk.argmax(axis=2)
    S = oracle.E4M3_VALUES[q.scales]
    normal = S >= 2.0 ** -6
    assert normal.sum() > 1000
    r, b = np.nonzero(normal)
    c = b * 16 + arg[r, b]
    assert ((codes[r, c] & 7) == 7).all()
    rel = np.abs(deq[r, c] - xf[r, c]) / np.abs(xf[r, c])
    assert rel.max() <= 2.0 ** -4
    # the block holding the tensor amax gets the largest scale, 448
    i = np.unravel_index(np.abs(xf).argmax(), xf.shape)
    assert q.scales[i[0], i[1] // 16] == 0x7E


def test_scaling_by_power_of_two_changes_only_s_enc():
    # I-5 (metamorphic): x * 2^k leaves codes and scales unchanged and multiplies
    # s_enc by 2^-k; x -> -x flips only the sign bits (RNE).
    rng = np.random.default_rng(4)
    x = _rand_bits(rng, (64, 128), "normal")
    q0 = oracle.quantize(x, oracle.BLOCK_1X16, oracle.RNE)
    for k in (-7, 3, 20):
        xk = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(x) * np.float32(2.0 ** k))
        qk = oracle.quantize(xk, oracle.BLOCK_1X16, oracle.RNE)
        np.testing.assert_array_equal(qk.codes, q0.codes)
        np.testing.assert_array_equal(qk.scales, q0.scales)
        assert qk.s_enc == q0.s_enc * 2.0 ** -k
    qn = oracle.quantize(x ^ np.uint16(0x8000), oracle.BLOCK_1X16, oracle.RNE)
    np.testing.assert_array_equal(qn.codes, q0.codes ^ np.uint8(0x88))
    np.testing.assert_array_equal(qn.scales, q0.scales)


def test_2d_blocks_transpose_invariance():
    # I-8 (2.B.3): quantising W^T with 16x16 blocks gives the transpose of the
    # quantised W -- the forward and backward passes see the same values.
    rng = np.random.default_rng(5)
    w = wl.normal(rng, (96, 160), 0.02)
    q = oracle.quantize(w, oracle.BLOCK_16X16, oracle.RNE)
    qt = oracle.quantize(np.ascontiguousarray(w.T), oracle.BLOCK_16X16, oracle.RNE)
    np.testing.assert_array_equal(oracle.unpack_codes(qt.codes, 96),
                                  oracle.unpack_codes(q.codes, 160).T)
    np.testing.assert_array_equal(qt.scales, q.scales.T)
    np.testing.assert_array_equal(oracle.dequantize(qt), oracle.dequantize(q).T)
    # 1x16 blocks do not have this property in general
    q1 = oracle.quantize(w, oracle.BLOCK_1X16, oracle.RNE)
    q1t = oracle.quantize(np.ascontiguousarray(w.T), oracle.BLOCK_1X16, oracle.RNE)
    assert not np.array_equal(oracle.dequantize(q1t), oracle.dequantize(q1).T)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_sr_unbiased(sign):
    # I-9 (2.B.4): over 10^6 draws the mean of the stochastically rounded value
    # is the input, within 5 standard errors plus the 2^-16 * gap resolution of
    # the 16-bit draw; every result is one of the two neighbours.
    n = 10 ** 6
    for seed in (1, 2, 3):
        u = oracle.sr_draws(seed, 0, n)
        for lo, g in [(0.0, 0.5), (0.5, 0.5), (1.5, 0.5), (2.0, 1.0), (3.0, 1.0), (4.0, 2.0)]:
            for r in (2.0 ** -10, 1 / 3, 0.5, 0.9):
                y = np.float32(sign * (lo + r * g))
                codes = oracle.e2m1_encode_sr(np.full(n, y, np.float32), u)
                vals = oracle.E2M1_VALUES[codes]
                assert set(np.unique(np.abs(vals))).issubset({lo, lo + g})
                rr = (abs(float(y)) - lo) / g
                se = g * np.sqrt(rr * (1 - rr) / n)
                assert abs(vals.mean() - float(y)) <= 5 * se + 2.0 ** -16 * g


def test_zero_and_underflow_blocks():
    # amax = 0 gives s_enc = 1 and all codes +-0; blocks far below the tensor amax
    # get a zero E4M3 scale and signed-zero codes.
    z = np.zeros((16, 32), np.uint16)
    z[3, 5] = 0x8000
    q = oracle.quantize(z, oracle.BLOCK_1X16, oracle.RNE)
    assert q.amax == 0.0 and q.s_enc == 1.0
    assert (q.scales == 0).all()
    codes = oracle.unpack_codes(q.codes, 32)
    assert codes[3, 5] == 8 and codes.sum() == 8
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1e4
    x[0, 16:] = np.linspace(-1e-5, 1e-5, 16)
    xb = wl.f32_to_bf16_bits(x)
    q = oracle.quantize(xb, oracle.BLOCK_1X16, oracle.RNE)
    assert q.scales[0, 1] == 0
    c = oracle.unpack_codes(q.codes, 32)[0, 16:]
    assert set(c.tolist()) <= {0, 8}
    assert (c[:8] == 8).all()


def test_amax_in_overrides():
    rng = np.random.default_rng(6)
    x = _rand_bits(rng, (32, 64), "normal")
    q = oracle.quantize(x, oracle.BLOCK_1X16, oracle.RNE)
    q2 = oracle.quantize(x, oracle.BLOCK_1X16, oracle.RNE, amax_in=q.amax)
    np.testing.assert_array_equal(q.codes, q2.codes)
    q3 = oracle.quantize(x, oracle.BLOCK_1X16, oracle.RNE, amax_in=2 * q.amax)
    assert q3.s_enc == np.float32(2688.0 / np.float32(2 * q.amax))


def test_nvfp4_error_below_mxfp4_style_scaling():
    # S-1 (sanity, not parity; 2.A): finer E4M3/16 scaling gives a lower
    # dequantisation error than power-of-two scales on 32-element blocks.
    rng = np.random.default_rng(8)
    x = _rand_bits(rng, (256, 512), "normal")
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    q = oracle.quantize(x, oracle.BLOCK_1X16, oracle.RNE)
    mse_nv = np.mean((oracle.dequantize(q) - xf) ** 2)
    # power-of-two scale per 32 elements: 2^ceil(log2(amax_b / 6)), RNE on the grid
    blk = xf.reshape(256, 16, 32)
    am = np.abs(blk).max(axis=2, keepdims=True)
    sc = 2.0 ** np.ceil(np.log2(am / 6))
    codes = oracle.e2m1_encode_rne((blk / sc).astype(np.float32))
    mse_mx = np.mean((oracle.E2M1_VALUES[codes] * sc - blk) ** 2)
    assert mse_nv < mse_mx


# --- slices of a larger tensor (sampled parity at full sizes) ---------------

def test_amax_helpers_match_quantisers():
    # the stand-alone maxima equal the ones the quantisers take themselves
    rng = np.random.default_rng(21)
    x = wl.lognormal_rows(rng, (48, 64))
    x[5, 7] = wl.f32_to_bf16_bits(np.array([-123.0], np.float32))[0]   # largest is negative
    assert oracle.amax(x) == oracle.quantize(x).amax == 123.0
    assert oracle.amax(x, rows_per_chunk=7) == 123.0
    mask = oracle.rht_sign_mask(4)
    want = oracle.rht_quantize(x, mask).amax
    assert oracle.rht_amax(x, mask) == want
    assert oracle.rht_amax(x, mask, channels_per_chunk=5) == want
    assert oracle.amax(np.zeros((0, 16), np.uint16)) == 0.0


def test_row_slices_with_index_offset_match_whole_tensor():
    # SR draws are indexed by the element's place in the whole tensor: a row
    # slice quantised with idx0 = r0 * cols and the whole tensor's amax gives
    # the same codes and scales as those rows of the whole result.
    rng = np.random.default_rng(22)
    rows, cols = 40, 96
    x = wl.lognormal_rows(rng, (rows, cols))
    full = oracle.quantize(x, rounding=oracle.SR, seed=77)
    for r0, r1 in [(0, 3), (17, 18), (33, 40)]:
        part = oracle.quantize(x[r0:r1], rounding=oracle.SR, seed=77, amax_in=full.amax,
                               idx0=r0 * cols)
        np.testing.assert_array_equal(part.codes, full.codes[r0:r1])
        np.testing.assert_array_equal(part.scales, full.scales[r0:r1])
        assert part.s_enc == full.s_enc
    # without the offset the draws differ (the slice is not the tensor's start)
    off = oracle.quantize(x[17:18], rounding=oracle.SR, seed=77, amax_in=full.amax)
    assert not np.array_equal(off.codes, full.codes[17:18])
    # 16x16 tiles: a column slice of whole tiles is independent of the rest
    w = wl.normal(rng, (32, 96), 0.02)
    fw = oracle.quantize(w, oracle.BLOCK_16X16)
    pw = oracle.quantize(np.ascontiguousarray(w[:, 32:64]), oracle.BLOCK_16X16, amax_in=fw.amax)
    np.testing.assert_array_equal(pw.codes, fw.codes[:, 16:32])
    np.testing.assert_array_equal(pw.scales, fw.scales[:, 2:4])


def test_channel_slices_with_index_offset_match_whole_rht_operand():
    rng = np.random.default_rng(23)
    tokens, channels = 64, 40
    x = wl.lognormal_rows(rng, (tokens, channels))
    mask = oracle.rht_sign_mask(9)
    full = oracle.rht_quantize(x, mask, oracle.SR, 5)
    for c0, c1 in [(0, 2), (13, 14), (37, 40)]:
        part = oracle.rht_quantize(np.ascontiguousarray(x[:, c0:c1]), mask, oracle.SR, 5,
                                   amax_in=full.amax, idx0=c0 * tokens)
        np.testing.assert_array_equal(part.codes, full.codes[c0:c1])
        np.testing.assert_array_equal(part.scales, full.scales[c0:c1])
