"""Pins of the oracle's random Hadamard transform and GEMM references.

RHT: "Pretraining Large Language Models with NVFP4", Technische
Zusammenfassung 2.B.2 -- a 16x16 Hadamard rotation, applied only to the inputs
of the weight-gradient GEMM.  GEMM: the three passes of a linear layer
(2.B.2 names Fprop, Dgrad and Wgrad).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from quantize_precision_gemm_amd import workloads as wl
from tests import exact_nvfp4 as ex


def hadamard16():
    """Sylvester Hadamard matrix from its closed form H[i][k] = (-1)^popcount(i & k)."""
    return np.array([[(-1) ** bin(i & k).count("1") for k in range(16)] for i in range(16)],
                    dtype=np.int64)


def test_hadamard_orthogonality():
    # I-7: H H^T = 16 I, exactly (integers)
    H = hadamard16()
    np.testing.assert_array_equal(H @ H.T, 16 * np.eye(16, dtype=np.int64))


def test_rht16_equals_matrix_form_on_integers():
    # On small integer vectors every butterfly sum is exact, so the transform must
    # equal (1/4) H D v exactly, for every position and sign pattern.
    H = hadamard16()
    rng = np.random.default_rng(0)
    for mask in [0, 1, 0x8000, 0xFFFF, 0x5A5A] + list(rng.integers(0, 65536, 20)):
        mask = int(mask)
        d = np.array([-1 if (mask >> i) & 1 else 1 for i in range(16)])
        for _ in range(10):
            v = rng.integers(-1000, 1000, 16)
            want = (H @ (d * v)) / 4.0
            got = oracle.rht16(v.astype(np.float32), mask)
            np.testing.assert_array_equal(got, want)
        for k in range(16):  # unit vectors give the columns of (1/4) H D
            e = np.zeros(16)
            e[k] = 1
            np.testing.assert_array_equal(oracle.rht16(e.astype(np.float32), mask),
                                          H[:, k] * d[k] / 4.0)


def test_rht16_inverts_and_is_close_to_exact():
    # Q = (1/4) H D is orthogonal: Q^T Q v = v.  On random fp32 data the fp32
    # butterfly stays within a few ulps of the exact transform.
    H = hadamard16().astype(np.float64)
    rng = np.random.default_rng(1)
    for _ in range(200):
        mask = int(rng.integers(0, 65536))
        d = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
        v = (rng.standard_normal(16) * np.exp(rng.uniform(-5, 5))).astype(np.float32)
        w = oracle.rht16(v, mask).astype(np.float64)
        exact = (H @ (d * v.astype(np.float64))) / 4
        scale = np.abs(v).astype(np.float64).sum() / 4
        assert np.abs(w - exact).max() <= 8 * 2.0 ** -24 * scale
        back = d * (H.T @ w) / 4
        np.testing.assert_allclose(back, v, rtol=0, atol=1e-6 * np.abs(v).max())


def test_rht_transform_preserves_wgrad_product():
    # (Q dY)^T (Q X) = dY^T X for the unquantised operands (fp32 tolerance).
    rng = np.random.default_rng(2)
    dy = wl.normal(rng, (64, 48), 1.0)
    x = wl.normal(rng, (64, 40), 1.0)
    mask = oracle.rht_sign_mask(5)
    A = oracle.rht_transform(dy, mask).astype(np.float64)   # 48 x 64
    B = oracle.rht_transform(x, mask).astype(np.float64)    # 40 x 64
    ref = wl.bf16_bits_to_f32(dy).astype(np.float64).T @ wl.bf16_bits_to_f32(x).astype(np.float64)
    np.testing.assert_allclose(A @ B.T, ref, rtol=0, atol=1e-5 * np.abs(ref).max())


def test_rht_quantize_brute_force():
    # The quantised wgrad operand equals the exact-arithmetic quantiser applied to
    # the oracle's fp32 transform (every transformed value is an fp32 number, so
    # it is fed to the exact model as such).
    rng = np.random.default_rng(3)
    x = wl.normal(rng, (32, 3), 1.0)
    mask = oracle.rht_sign_mask(9)
    for rounding in (oracle.RNE, oracle.SR):
        q = oracle.rht_quantize(x, mask, rounding, seed=77)
        t = oracle.rht_transform(x, mask)  # 3 x 32 fp32
        flat = [Fraction(float(v)) for v in t.reshape(-1)]
        amax = max(abs(v) for v in flat)
        assert np.float32(q.amax) == np.float32(float(amax))
        s_enc = ex.tensor_scale(amax)
        assert np.float32(q.s_enc) == np.float32(float(s_enc))
        draws = oracle.sr_draws(77, 0, len(flat))
        codes = oracle.unpack_codes(q.codes, 32).reshape(-1)
        for b in range(len(flat) // 16):
            blk = flat[16 * b: 16 * b + 16]
            am = max(abs(v) for v in blk)
            sb = ex.nearest_e4m3(ex.round_f32(ex.round_f32(am / 6) * s_enc))
            assert q.scales.reshape(-1)[b] == sb
            S = ex.E4M3_VAL[sb]
            f = ex.round_f32(s_enc / S) if S > 0 else Fraction(0)
            for i, v in enumerate(blk):
                y = ex.round_f32(abs(v) * f)
                c = ex.nearest_e2m1_code(y) if rounding == oracle.RNE else \
                    ex.sr_e2m1_code(y, int(draws[16 * b + i]))
                sign = 8 if np.signbit(t.reshape(-1)[16 * b + i]) else 0
                assert codes[16 * b + i] == (sign | c)


def _exact_value(q, r, k):
    """Exact decoded value q * S of element (r, k) of an NVFP4 tensor, read
    straight from its packed codes and scale bytes through the exact model's
    value lists (no oracle decode table): code = nibble k % 2 of byte k / 2
    (low nibble first), scale byte at (r, k / 16) for 1x16 blocks and at
    (r / 16, k / 16) for 16x16 blocks."""
    byte = int(q.codes[r, k // 2])
    c = (byte >> 4) if k % 2 else (byte & 0xF)
    sb = int(q.scales[r, k // 16] if q.block == oracle.BLOCK_1X16 else q.scales[r // 16, k // 16])
    mag = ex.E2M1_MAGS[c & 7] * ex.E4M3_VAL[sb]
    return -mag if c & 8 else mag


def _exact_gemm(a, b, dgrad=False):
    """Exact rational GEMM of the dequantised operands, (q * S) / s_enc.
    fprop/wgrad: C[m, n] = sum_k A[m, k] B[n, k]; dgrad: C[m, k] = sum_n A[m, n] B[n, k]."""
    alpha = Fraction(1) / (Fraction(a.s_enc) * Fraction(b.s_enc))
    M = a.rows
    if dgrad:
        N, red = b.cols, a.cols
        term = lambda m, n, j: _exact_value(a, m, j) * _exact_value(b, j, n)
    else:
        N, red = b.rows, a.cols
        term = lambda m, n, j: _exact_value(a, m, j) * _exact_value(b, n, j)
    out = np.empty((M, N))
    for m in range(M):
        for n in range(N):
            out[m, n] = float(sum(term(m, n, j) for j in range(red)) * alpha)
    return out


def test_decode_tables_match_exact_model():
    # The fp64 decode tables every oracle GEMM and dequantisation multiplies by
    # (Technische Zusammenfassung 2.A: E2M1 elements, E4M3 block scales) equal
    # the exact model's value lists entry by entry: all 16 E2M1 codes, and all
    # 127 finite E4M3 bytes of each sign, including the subnormal scale bytes
    # 0x01-0x07 (m * 2^-9).
    for c in range(16):
        want = ex.E2M1_MAGS[c & 7]
        assert Fraction(float(oracle.E2M1_VALUES[c])) == (-want if c & 8 else want)
        assert np.signbit(oracle.E2M1_VALUES[c]) == bool(c & 8)
    for b, v in ex.E4M3_LIST:
        assert Fraction(float(oracle.E4M3_VALUES[b])) == v, hex(b)
        assert Fraction(float(oracle.E4M3_VALUES[0x80 | b])) == -v, hex(0x80 | b)
    assert [float(oracle.E4M3_VALUES[b]) for b in range(1, 8)] == [m / 512 for m in range(1, 8)]
    assert np.isnan(oracle.E4M3_VALUES[0x7F]) and np.isnan(oracle.E4M3_VALUES[0xFF])


def _rows_scaled(rng, shape, factors):
    """bf16 rows ~N(0, 1) times per-row factors (spans E4M3's subnormal and zero scales)."""
    x = rng.standard_normal(shape) * np.asarray(factors, np.float64)[:, None]
    return wl.f32_to_bf16_bits(x.astype(np.float32))


def test_gemm_reference_matches_exact_rationals():
    # I-10 (exactness part): the fp64 reference equals the exact product of the
    # dequantised operands (decoded independently of the oracle's tables) to
    # fp64 rounding, for all three passes.
    rng = np.random.default_rng(4)
    x = wl.normal(rng, (4, 32), 1.0)
    w = wl.normal(rng, (16, 32), 0.02)
    dy = wl.lognormal_rows(rng, (4, 16))
    qx = oracle.quantize(x)
    qw = oracle.quantize(w, oracle.BLOCK_16X16)
    qdy = oracle.quantize(dy, rounding=oracle.SR, seed=3)
    y = oracle.gemm(oracle.FPROP, qx, qw)
    np.testing.assert_allclose(y, _exact_gemm(qx, qw), rtol=1e-13, atol=0)
    dx = oracle.gemm(oracle.DGRAD, qdy, qw)
    np.testing.assert_allclose(dx, _exact_gemm(qdy, qw, dgrad=True), rtol=1e-13, atol=0)
    mask = oracle.rht_sign_mask(1)
    dyt = oracle.rht_quantize(wl.normal(rng, (32, 4), 1.0), mask, oracle.SR, 5)
    xt = oracle.rht_quantize(wl.normal(rng, (32, 5), 1.0), mask, oracle.RNE)
    dw = oracle.gemm(oracle.WGRAD, dyt, xt)
    np.testing.assert_allclose(dw, _exact_gemm(dyt, xt), rtol=1e-13, atol=0)


@pytest.mark.parametrize("rounding", [oracle.RNE, oracle.SR])
def test_gemm_reference_exact_with_subnormal_block_scales(rounding):
    # Blocks whose E4M3 scale is subnormal (bytes 0x01-0x07) or zero: rows
    # 1e-4 .. 1e-7 of the tensor's largest row (block scale ~448 * ratio, so
    # 2^-9 .. 2^-6 is subnormal, below 2^-10 rounds to zero).  A wrong
    # subnormal decode entry changes these rows of the product.
    rng = np.random.default_rng(40)
    factors = [1.0, 3e-5, 1e-5, 4e-6, 1.5e-6, 1e-7]
    a = oracle.quantize(_rows_scaled(rng, (6, 48), factors), rounding=rounding, seed=11)
    b = oracle.quantize(_rows_scaled(rng, (5, 48), [1.0, 2e-5, 7e-6, 1.0, 2e-6]), rounding=rounding, seed=12)
    sub_a = set(int(v) for v in a.scales.reshape(-1) if 0 < v < 8)
    sub_b = set(int(v) for v in b.scales.reshape(-1) if 0 < v < 8)
    assert len(sub_a) >= 3 and len(sub_b) >= 2, (sub_a, sub_b)  # the case is exercised
    assert (a.scales == 0).any()
    got = oracle.gemm(oracle.WGRAD, a, b)  # C = A B^T over 1x16 blocks
    want = _exact_gemm(a, b)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=0)
    # the subnormal-scale rows are not negligible in their own outputs
    assert np.all(np.abs(want[1:5, 1:3]) > 0)


def test_gemm_fp32_accumulation_within_budget():
    # I-10 (tolerance part): an fp32 GEMM that sums exact 16-block partials in
    # order stays within 1e-6 relative Frobenius of the fp64 reference at the
    # longest contraction of the layer shapes (20480), well inside the 1e-5 budget.
    rng = np.random.default_rng(5)
    K = 20480
    a = oracle.quantize(wl.lognormal_rows(rng, (8, K)), rounding=oracle.SR, seed=9)
    b = oracle.quantize(wl.normal(rng, (32, K), 0.02), oracle.BLOCK_16X16)
    ref = oracle.gemm(oracle.FPROP, a, b)
    f32 = oracle.gemm_fp32_blocks(a, b).astype(np.float64)
    err = np.linalg.norm(f32 - ref) / np.linalg.norm(ref)
    assert err < 1e-6


def test_gemm_sampled_rows_match_full():
    rng = np.random.default_rng(6)
    a = oracle.quantize(wl.normal(rng, (40, 64), 1.0))
    b = oracle.quantize(wl.normal(rng, (32, 64), 0.02), oracle.BLOCK_16X16)
    full = oracle.gemm(oracle.FPROP, a, b)
    rows = np.array([0, 7, 39])
    np.testing.assert_array_equal(oracle.gemm(oracle.FPROP, a, b, rows=rows), full[rows])


# --- bf16 GEMM of the layers kept in high precision (Technische
# Zusammenfassung 2.B.1; passes of 2.B.2) ------------------------------------

def test_bf16_bits_decode_closed_forms():
    cases = {0x3F80: 1.0, 0xBF80: -1.0, 0x4049: 3.140625, 0x0001: 2.0 ** -133,
             0x0080: 2.0 ** -126, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x0000: 0.0,
             0xC2F7: -123.5}
    bits = np.array(list(cases), dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    np.testing.assert_array_equal(got, np.array(list(cases.values())))
    assert np.signbit(oracle.bf16_bits_to_f64(np.array([0x8000], dtype=np.uint16)))[0]


def test_bf16_bits_decode_matches_torch():
    # torch's own bfloat16 -> float64 conversion on every finite bit pattern
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite]
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(bits), ref)


def _bf16_value(u):
    s, mag = ex.bf16_bits_to_fraction(int(u))
    return -mag if s else mag


@pytest.mark.parametrize("pass_", [oracle.FPROP, oracle.DGRAD, oracle.WGRAD])
def test_bf16_gemm_passes_brute_force(pass_):
    # Each pass written out with explicit indices over exact rationals: a
    # transposed operand or a swapped pass would fail here.
    rng = np.random.default_rng(10 + pass_)
    M, N, K = 3, 5, 4
    x = wl.normal(rng, (M, K), 1.0)
    w = wl.normal(rng, (N, K), 0.02)
    dy = wl.lognormal_rows(rng, (M, N))
    X = [[_bf16_value(v) for v in r] for r in x]
    W = [[_bf16_value(v) for v in r] for r in w]
    DY = [[_bf16_value(v) for v in r] for r in dy]
    if pass_ == oracle.FPROP:
        got = oracle.bf16_gemm(pass_, x, w)
        ref = [[sum(X[m][k] * W[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
    elif pass_ == oracle.DGRAD:
        got = oracle.bf16_gemm(pass_, dy, w)
        ref = [[sum(DY[m][n] * W[n][k] for n in range(N)) for k in range(K)] for m in range(M)]
    else:
        got = oracle.bf16_gemm(pass_, dy, x)
        ref = [[sum(DY[m][n] * X[m][k] for m in range(M)) for k in range(K)] for n in range(N)]
    ref = np.array([[float(v) for v in r] for r in ref])
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=0)


@pytest.mark.parametrize("pass_", [oracle.FPROP, oracle.DGRAD, oracle.WGRAD])
def test_bf16_gemm_sampled_rows_match_full(pass_):
    rng = np.random.default_rng(11)
    M, N, K = 24, 16, 40
    x = wl.normal(rng, (M, K), 1.0)
    w = wl.normal(rng, (N, K), 0.02)
    dy = wl.normal(rng, (M, N), 1.0)
    a, b = {oracle.FPROP: (x, w), oracle.DGRAD: (dy, w), oracle.WGRAD: (dy, x)}[pass_]
    full = oracle.bf16_gemm(pass_, a, b)
    rows = np.array([0, 3, full.shape[0] - 1])
    np.testing.assert_array_equal(oracle.bf16_gemm(pass_, a, b, rows=rows), full[rows])


def _scaled_bits(u16, k):
    """bf16 bit patterns times 2^k (exact: exponent field shift, no under/overflow here)."""
    return wl.f32_to_bf16_bits((wl.bf16_bits_to_f32(u16).astype(np.float64) * 2.0 ** k).astype(np.float32))


@pytest.mark.parametrize("k", [-40, -52, -55])
def test_gemm_fp32_output_scale_below_normal_range(k):
    # Both operands times 2^k: codes and scales stay (I-5), each tensor scale
    # gains 2^-k, so the product of the two FP32 decode scales loses 2^2k and,
    # for k = -52 / -55, falls below fp32's normal range (amax product <
    # ~8.5e-32) while every output stays a normal number.  The fp32 block
    # GEMM's output is then exactly the unscaled output times 2^2k, and within
    # 1e-6 of the fp64 reference.
    rng = np.random.default_rng(41)
    x = wl.normal(rng, (8, 64), 1.0)
    w = wl.normal(rng, (16, 64), 0.02)
    a, b = oracle.quantize(x), oracle.quantize(w, oracle.BLOCK_16X16)
    a2, b2 = oracle.quantize(_scaled_bits(x, k)), oracle.quantize(_scaled_bits(w, k), oracle.BLOCK_16X16)
    np.testing.assert_array_equal(a2.codes, a.codes)
    np.testing.assert_array_equal(b2.scales, b.scales)
    alpha32 = np.float32(np.float32(1) / a2.s_enc) * np.float32(np.float32(1) / b2.s_enc)
    if k <= -52:
        assert alpha32 < np.finfo(np.float32).tiny  # the case is exercised
    base = oracle.gemm_fp32_blocks(a, b).astype(np.float64)
    got = oracle.gemm_fp32_blocks(a2, b2).astype(np.float64)
    assert np.all(np.abs(got[got != 0]) >= np.finfo(np.float32).tiny)
    np.testing.assert_array_equal(got, base * 2.0 ** (2 * k))
    ref = oracle.gemm(oracle.FPROP, a2, b2)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-6
