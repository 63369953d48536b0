"""Pins of the oracle's sized random Hadamard transform (sizes 4, 16, 64):
the ablation of the 16 x 16 choice in "Pretraining Large Language Models
with NVFP4", Technische Zusammenfassung 2.B.2.  Checked against the
Sylvester closed form on integer vectors, the established 16-point
functions, the inverse transform, and an independent matrix-form
quantisation of the transformed tensor."""
import numpy as np
import pytest

import oracle
from quantize_precision_gemm_amd import workloads as wl


def hadamard(D):
    return np.array([[(-1) ** bin(i & k).count("1") for k in range(D)] for i in range(D)],
                    dtype=np.int64)


def test_signs64_extend_the_16_point_signs():
    for seed in [0, 7, 1000, 2 ** 40 + 3]:
        s = oracle.rht_signs64(seed)
        assert s & 0xFFFF == oracle.rht_sign_mask(seed)
        w = oracle.philox4x32_10([0, 0, 0, 1], [seed & 0xFFFFFFFF, seed >> 32])
        assert s == int(w[0]) | (int(w[1]) << 32)


def test_size16_is_the_established_transform():
    rng = np.random.default_rng(1)
    for _ in range(50):
        v = rng.standard_normal(16).astype(np.float32) * np.float32(10 ** rng.uniform(-3, 3))
        m = int(rng.integers(0, 2 ** 63))
        np.testing.assert_array_equal(oracle.rht_sized(v, 16, m), oracle.rht16(v, m & 0xFFFF))


@pytest.mark.parametrize("D", [4, 16, 64])
def test_matrix_form_on_integers(D):
    # (1/sqrt D) H_D diag(d) v, exact for small integer v (every partial sum
    # is an integer below 2^24 and the normalisation a power of two)
    rng = np.random.default_rng(D)
    H = hadamard(D)
    for _ in range(20):
        v = rng.integers(-1000, 1001, D)
        signs = int(rng.integers(0, 2 ** 63)) | (int(rng.integers(0, 2)) << 63)
        d = np.array([-1 if (signs >> i) & 1 else 1 for i in range(D)], np.int64)
        want = (H @ (d * v)).astype(np.float64) / np.sqrt(D)
        got = oracle.rht_sized(v.astype(np.float32), D, signs)
        np.testing.assert_array_equal(got.astype(np.float64), want)


@pytest.mark.parametrize("D", [4, 64])
def test_inverse(D):
    # H D_s v / sqrt(D) transformed again with no signs gives D_s v
    rng = np.random.default_rng(10 + D)
    v = rng.integers(-500, 501, D).astype(np.float32)
    signs = int(rng.integers(0, 2 ** 63))
    back = oracle.rht_sized(oracle.rht_sized(v, D, signs), D, 0)
    d = np.array([-1 if (signs >> i) & 1 else 1 for i in range(D)], np.float32)
    np.testing.assert_array_equal(back, d * v)


@pytest.mark.parametrize("rounding", [0, 1])
def test_sized16_quantiser_equals_rht_quantize(rounding):
    rng = np.random.default_rng(20 + rounding)
    x = wl.lognormal_rows(rng, (96, 40))
    s = oracle.rht_signs64(3)
    a = oracle.rht_quantize_sized(x, 16, s, rounding, 9)
    b = oracle.rht_quantize(x, s & 0xFFFF, rounding, 9)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.scales, b.scales)
    assert a.amax == b.amax and a.s_enc == b.s_enc


@pytest.mark.parametrize("D", [4, 64])
@pytest.mark.parametrize("rounding", [0, 1])
def test_sized_quantiser_equals_quantised_matrix_form(D, rounding):
    # integer inputs: the transform (Sylvester form, numpy) is exact and
    # bf16-representable, so quantising its transpose with the plain 1x16
    # quantiser -- whose SR index r * tokens + t is the wgrad layout's --
    # gives the sized quantiser's codes, scales and tensor scale
    rng = np.random.default_rng(30 + D + rounding)
    tokens, channels = 128, 24
    xi = rng.integers(-6, 7, (tokens, channels))
    x = wl.f32_to_bf16_bits(xi.astype(np.float32))
    signs = oracle.rht_signs64(11)
    d = np.array([-1 if (signs >> i) & 1 else 1 for i in range(D)], np.int64)
    H = hadamard(D)
    T = np.empty((tokens, channels), np.float64)
    for j in range(tokens // D):
        T[D * j:D * j + D] = (H @ (d[:, None] * xi[D * j:D * j + D])) / np.sqrt(D)
    tb = wl.f32_to_bf16_bits(T.astype(np.float32))
    assert np.array_equal(wl.bf16_bits_to_f32(tb).astype(np.float64), T)
    want = oracle.quantize(np.ascontiguousarray(tb.T), oracle.BLOCK_1X16, rounding, 5)
    got = oracle.rht_quantize_sized(x, D, signs, rounding, 5)
    # element values, not code bytes: where the transform is exactly zero the
    # butterfly can give -0 (-0 + -0 after two sign flips) and the integer
    # matrix form +0; both quantise to a zero
    gv = oracle.E2M1_VALUES[oracle.unpack_codes(got.codes, tokens)]
    wv = oracle.E2M1_VALUES[oracle.unpack_codes(want.codes, tokens)]
    np.testing.assert_array_equal(gv, wv)
    np.testing.assert_array_equal(got.scales, want.scales)
    assert got.amax == want.amax and got.s_enc == want.s_enc


def test_shapes_and_sizes_checked():
    x = np.zeros((48, 8), np.uint16)
    with pytest.raises(ValueError):
        oracle.rht_quantize_sized(x, 64, 0)      # 48 tokens: not whole 64-token chunks
    with pytest.raises(ValueError):
        oracle.rht_quantize_sized(x, 8, 0)       # size 8: normalisation not a power of two


@pytest.mark.parametrize("rounding", [0, 1])
def test_size1_is_the_plain_transposed_quantiser(rounding):
    # no transform: the wgrad operand is the 1x16 quantisation of x^T, whose
    # SR index r * tokens + t is the same as the sized quantiser's
    rng = np.random.default_rng(40 + rounding)
    x = wl.lognormal_rows(rng, (64, 40))
    got = oracle.rht_quantize_sized(x, 1, 0, rounding, 8)
    want = oracle.quantize(np.ascontiguousarray(x.T), oracle.BLOCK_1X16, rounding, 8)
    np.testing.assert_array_equal(got.codes, want.codes)
    np.testing.assert_array_equal(got.scales, want.scales)
    assert got.amax == want.amax


# --- RHT along the rows: the fprop / dgrad operands --------------------------

@pytest.mark.parametrize("block", [0, 1])
@pytest.mark.parametrize("rounding", [0, 1])
def test_row_rht_quantiser_equals_quantised_matrix_form(block, rounding):
    # integer inputs: the per-chunk transform (Sylvester form) is exact and
    # bf16-representable, so the plain quantiser applied to it gives the same
    # codes (as values: exact zeros may carry either sign), scales and scale
    rng = np.random.default_rng(50 + 2 * block + rounding)
    rows, cols = 48, 96
    xi = rng.integers(-6, 7, (rows, cols))
    x = wl.f32_to_bf16_bits(xi.astype(np.float32))
    mask = oracle.rht_sign_mask(13)
    d = np.array([-1 if (mask >> i) & 1 else 1 for i in range(16)], np.int64)
    H = hadamard(16)
    T = (xi.reshape(rows, cols // 16, 16) * d) @ H.T / 4.0      # H symmetric: row chunk v -> H D v
    tb = wl.f32_to_bf16_bits(T.reshape(rows, cols).astype(np.float32))
    assert np.array_equal(wl.bf16_bits_to_f32(tb).astype(np.float64), T.reshape(rows, cols))
    want = oracle.quantize(tb, block, rounding, 3)
    got = oracle.quantize_rht_rows(x, mask, block, rounding, 3)
    gv = oracle.E2M1_VALUES[oracle.unpack_codes(got.codes, cols)]
    wv = oracle.E2M1_VALUES[oracle.unpack_codes(want.codes, cols)]
    np.testing.assert_array_equal(gv, wv)
    np.testing.assert_array_equal(got.scales, want.scales)
    assert got.amax == want.amax and got.s_enc == want.s_enc


def test_row_rht_preserves_the_product():
    # one sign vector for both operands: the transforms cancel in A B^T
    rng = np.random.default_rng(60)
    a = wl.f32_to_bf16_bits(rng.integers(-8, 9, (8, 64)).astype(np.float32))
    b = wl.f32_to_bf16_bits(rng.integers(-8, 9, (5, 64)).astype(np.float32))
    mask = oracle.rht_sign_mask(2)
    ta = np.concatenate([oracle.rht16(wl.bf16_bits_to_f32(a)[r, 16 * j:16 * j + 16], mask)
                         for r in range(8) for j in range(4)]).reshape(8, 64).astype(np.float64)
    tb = np.concatenate([oracle.rht16(wl.bf16_bits_to_f32(b)[r, 16 * j:16 * j + 16], mask)
                         for r in range(5) for j in range(4)]).reshape(5, 64).astype(np.float64)
    exact = wl.bf16_bits_to_f32(a).astype(np.float64) @ wl.bf16_bits_to_f32(b).astype(np.float64).T
    np.testing.assert_array_equal(ta @ tb.T, exact)
