"""GPU parity of the NVFP4 GEMM (fprop, dgrad, wgrad) against the fp64 oracle.

Bar: relative Frobenius error <= 1e-5 on the kernel's fp32 output; the bf16
output is bit-equal to round-to-nearest-even of that fp32 output.  Both
datapaths are checked: nvfp4_gemm (fp16 decode) and nvfp4_gemm_fp8blk (FP8
MFMA per block).  The latter sums exact block partials in block order, which
is what the oracle's fp32 block GEMM does, so it must match that bit for bit.
Passes: "Pretraining Large Language Models with NVFP4" (gist.science
summary), Technische Zusammenfassung 2.B.2 (Fprop, Dgrad, Wgrad).
"""
import numpy as np
import pytest

from tests.gpu_util import bf16_rne_bits, ensure_built, rel_fro, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module")
def env():
    import torch
    ensure_built()
    import oracle
    import quantize_precision_gemm_amd as q
    from quantize_precision_gemm_amd import workloads as wl
    dev = torch.device("cuda:0")
    return torch, oracle, q, wl, dev


def _check_both_dtypes(torch, q, pass_, ga, gb, want):
    out = None
    for fp8 in (False, True):
        y32 = q.nvfp4_gemm(pass_, ga, gb, torch.float32, fp8_blocks=fp8)
        y16 = q.nvfp4_gemm(pass_, ga, gb, torch.bfloat16, fp8_blocks=fp8)
        torch.cuda.synchronize()
        g32 = y32.cpu().numpy()
        err = rel_fro(g32, want)
        assert err <= TOL, f"{'fp8 blocks' if fp8 else 'fp16 decode'}: relative Frobenius error {err:.3e}"
        b16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
        np.testing.assert_array_equal(b16, bf16_rne_bits(g32))
        out = g32 if out is None else out
    return out


# (M, K, N): several 256-tiles, ragged M/N, K tails (K % 128 != 0, K % 32 == 16)
SHAPES = [(1, 16, 16), (16, 48, 32), (300, 336, 272), (257, 1040, 528), (512, 512, 768),
          (64, 4112, 96)]


@pytest.mark.parametrize("shape", SHAPES)
def test_fprop(env, shape):
    torch, oracle, q, wl, dev = env
    M, K, N = shape
    rng = np.random.default_rng(M + K + N)
    x = wl.student_t_unit_var(rng, (M, K), 4)
    w = wl.normal(rng, (N, K), 0.02)
    print(f"fprop {shape}", flush=True)
    gx = q.nvfp4_quantize(to_dev(x, dev), q.BLOCK_1X16, q.RNE)
    gw = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE, with_transpose=True)
    want = oracle.gemm(oracle.FPROP, oracle.quantize(x), oracle.quantize(w, oracle.BLOCK_16X16))
    _check_both_dtypes(torch, q, q.FPROP, gx, gw, want)
    # a 1x16-quantised B operand takes the same path with per-row scales
    gw1 = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_1X16, q.RNE)
    want1 = oracle.gemm(oracle.FPROP, oracle.quantize(x), oracle.quantize(w))
    _check_both_dtypes(torch, q, q.FPROP, gx, gw1, want1)


@pytest.mark.parametrize("shape", SHAPES)
def test_dgrad(env, shape):
    torch, oracle, q, wl, dev = env
    M, K, N = shape  # dX (M x K) = dY (M x N) W (N x K)
    rng = np.random.default_rng(3 * M + K + N)
    dy = wl.lognormal_rows(rng, (M, N))
    w = wl.normal(rng, (N, K), 0.02)
    print(f"dgrad {shape}", flush=True)
    gdy = q.nvfp4_quantize(to_dev(dy, dev), q.BLOCK_1X16, q.SR, 17)
    gw = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE, with_transpose=True)
    want = oracle.gemm(oracle.DGRAD, oracle.quantize(dy, oracle.BLOCK_1X16, oracle.SR, 17),
                       oracle.quantize(w, oracle.BLOCK_16X16))
    _check_both_dtypes(torch, q, q.DGRAD, gdy, gw, want)


@pytest.mark.parametrize("shape", [(16, 16, 16), (48, 40, 24), (272, 264, 200), (1040, 512, 264)])
def test_wgrad(env, shape):
    torch, oracle, q, wl, dev = env
    M, K, N = shape  # dW (N x K) = sum over M tokens
    rng = np.random.default_rng(5 * M + K + N)
    dy = wl.lognormal_rows(rng, (M, N))
    x = wl.student_t_unit_var(rng, (M, K), 4)
    mask = q.nvfp4_rht_sign_mask(M)
    print(f"wgrad {shape}", flush=True)
    gdyt = q.nvfp4_rht_quantize(to_dev(dy, dev), mask, q.SR, 23)
    gxt = q.nvfp4_rht_quantize(to_dev(x, dev), mask, q.RNE)
    want = oracle.gemm(oracle.WGRAD, oracle.rht_quantize(dy, mask, oracle.SR, 23),
                       oracle.rht_quantize(x, mask, oracle.RNE))
    _check_both_dtypes(torch, q, q.WGRAD, gdyt, gxt, want)


# Contraction lengths around the kernel's switch between one scale load per
# 64-element K step and one per three steps (taken while 9 or more whole
# steps remain): 8 to 16 whole steps, with and without a partial last step.
@pytest.mark.parametrize("K", [512, 528, 576, 592, 640, 704, 768, 960, 976, 1024])
def test_scale_load_switch(env, K):
    torch, oracle, q, wl, dev = env
    M, N = 264, 272
    rng = np.random.default_rng(K)
    x = wl.student_t_unit_var(rng, (M, K), 4)
    w = wl.normal(rng, (N, K), 0.02)
    dy = wl.lognormal_rows(rng, (M, K))
    print(f"scale-load switch K={K}", flush=True)
    gx = q.nvfp4_quantize(to_dev(x, dev), q.BLOCK_1X16, q.RNE)
    gw = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE, with_transpose=True)
    want = oracle.gemm(oracle.FPROP, oracle.quantize(x), oracle.quantize(w, oracle.BLOCK_16X16))
    _check_both_dtypes(torch, q, q.FPROP, gx, gw, want)
    # dgrad contracts over W's rows: here dY is M x K and W^T is read (K rows)
    w2 = wl.normal(rng, (K, N), 0.02)
    gdy = q.nvfp4_quantize(to_dev(dy, dev), q.BLOCK_1X16, q.SR, 5)
    gw2 = q.nvfp4_quantize(to_dev(w2, dev), q.BLOCK_16X16, q.RNE, with_transpose=True)
    want = oracle.gemm(oracle.DGRAD, oracle.quantize(dy, oracle.BLOCK_1X16, oracle.SR, 5),
                       oracle.quantize(w2, oracle.BLOCK_16X16))
    _check_both_dtypes(torch, q, q.DGRAD, gdy, gw2, want)


def test_wgrad_rht_cancels(env):
    # With the same sign mask on both operands the transform cancels in the
    # product: the NVFP4 wgrad stays close to the unquantised dY^T X.
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(9)
    M, K, N = 1024, 64, 96
    dy = wl.normal(rng, (M, N), 1.0)
    x = wl.normal(rng, (M, K), 1.0)
    mask = q.nvfp4_rht_sign_mask(4)
    gdyt = q.nvfp4_rht_quantize(to_dev(dy, dev), mask, q.SR, 1)
    gxt = q.nvfp4_rht_quantize(to_dev(x, dev), mask, q.RNE)
    dw = q.nvfp4_gemm(q.WGRAD, gdyt, gxt, torch.float32)
    torch.cuda.synchronize()
    ref = wl.bf16_bits_to_f32(dy).astype(np.float64).T @ wl.bf16_bits_to_f32(x).astype(np.float64)
    assert rel_fro(dw.cpu().numpy(), ref) < 0.2  # 4-bit quantisation noise, not a parity bar


def test_empty_contraction_and_determinism(env):
    torch, oracle, q, wl, dev = env
    a = q.alloc_nvfp4(32, 0)
    b = q.alloc_nvfp4(48, 0)
    a.amax.fill_(0)
    a.s_enc.fill_(1)
    b.s_enc.fill_(1)
    y = q.nvfp4_gemm(q.FPROP, a, b, torch.float32)
    torch.cuda.synchronize()
    assert (y == 0).all()
    rng = np.random.default_rng(1)
    x = to_dev(wl.normal(rng, (700, 640), 1.0), dev)
    w = to_dev(wl.normal(rng, (528, 640), 0.02), dev)
    gx = q.nvfp4_quantize(x)
    gw = q.nvfp4_quantize(w, q.BLOCK_16X16, q.RNE, with_transpose=True)
    y1 = q.nvfp4_gemm(q.FPROP, gx, gw, torch.float32)
    y2 = q.nvfp4_gemm(q.FPROP, gx, gw, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("shape", [(16, 16, 16), (300, 336, 272), (257, 1040, 528), (64, 4112, 96)])
@pytest.mark.parametrize("pass_name", ["fprop", "dgrad", "wgrad"])
def test_fp8blk_matches_block_oracle_bitwise(env, pass_name, shape):
    torch, oracle, q, wl, dev = env
    M, K, N = shape
    rng = np.random.default_rng(11 * M + K + N)
    print(f"fp8blk {pass_name} {shape}", flush=True)
    if pass_name == "fprop":
        x = wl.student_t_unit_var(rng, (M, K), 4)
        w = wl.normal(rng, (N, K), 0.02)
        ga = q.nvfp4_quantize(to_dev(x, dev))
        gb = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE, with_transpose=True)
        oa, ob = oracle.quantize(x), oracle.quantize(w, oracle.BLOCK_16X16)
        pass_ = q.FPROP
    elif pass_name == "dgrad":
        dy = wl.lognormal_rows(rng, (M, N))
        w = wl.normal(rng, (N, K), 0.02)
        ga = q.nvfp4_quantize(to_dev(dy, dev), q.BLOCK_1X16, q.SR, 3)
        gb = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE, with_transpose=True)
        # the block GEMM takes both operands rows x K: W^T quantised 16x16
        oa = oracle.quantize(dy, oracle.BLOCK_1X16, oracle.SR, 3)
        ob = oracle.quantize(np.ascontiguousarray(w.T), oracle.BLOCK_16X16)
        pass_ = q.DGRAD
    else:
        Mt = ((M + 15) // 16) * 16
        dy = wl.lognormal_rows(rng, (Mt, N))
        x = wl.student_t_unit_var(rng, (Mt, K), 4)
        mask = q.nvfp4_rht_sign_mask(Mt)
        ga = q.nvfp4_rht_quantize(to_dev(dy, dev), mask, q.SR, 5)
        gb = q.nvfp4_rht_quantize(to_dev(x, dev), mask, q.RNE)
        oa = oracle.rht_quantize(dy, mask, oracle.SR, 5)
        ob = oracle.rht_quantize(x, mask, oracle.RNE)
        pass_ = q.WGRAD
    y = q.nvfp4_gemm(pass_, ga, gb, torch.float32, fp8_blocks=True)
    torch.cuda.synchronize()
    want = oracle.gemm_fp32_blocks(oa, ob)
    got = y.cpu().numpy()
    assert got.shape == want.shape
    bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
    assert len(bad) == 0, f"{len(bad)} outputs differ, first {bad[0]}: {got[tuple(bad[0])]} vs {want[tuple(bad[0])]}"


@pytest.mark.parametrize("fp8", [False, True])
def test_padded_leading_dimensions(env, fp8):
    # Codes and scales with rows wider than needed, and an output with a wider
    # row: the quantisers and both GEMM datapaths honour every leading
    # dimension, and nothing past the logical columns of the output is written.
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(17)
    M, K, N = 272, 336, 208
    x = wl.student_t_unit_var(rng, (M, K), 4)
    w = wl.normal(rng, (N, K), 0.02)
    print(f"padded ld fp8={fp8}", flush=True)

    def padded(rows, cols, block, with_t):
        t = q.alloc_nvfp4(rows, cols, block, with_t, dev)
        srows = rows if block == q.BLOCK_1X16 else rows // 16
        t.codes = torch.empty((rows, t.codes.shape[1] + 48), dtype=torch.uint8, device=dev)
        t.scales = torch.empty((srows, t.scales.shape[1] + 8), dtype=torch.uint8, device=dev)
        return t

    gx = q.nvfp4_quantize(to_dev(x, dev), out=padded(M, K, q.BLOCK_1X16, False))
    gw = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE,
                          out=padded(N, K, q.BLOCK_16X16, True))
    assert gx.codes.stride(0) > K // 2 and gw.codes.stride(0) > K // 2
    want = oracle.gemm(oracle.FPROP, oracle.quantize(x), oracle.quantize(w, oracle.BLOCK_16X16))
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        buf = torch.full((M, N + 24), -3.0, dtype=dt, device=dev)
        q.nvfp4_gemm(q.FPROP, gx, gw, out=buf[:, :N], fp8_blocks=fp8)
        torch.cuda.synchronize()
        assert (buf[:, N:] == -3.0).all().item()
        outs[dt] = buf[:, :N].contiguous()
    g32 = outs[torch.float32].cpu().numpy()
    assert rel_fro(g32, want) <= TOL
    b16 = outs[torch.bfloat16].view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(b16, bf16_rne_bits(g32))


@pytest.mark.parametrize("case", ["ldc % 8 == 4", "8-byte aligned view", "N % 8 == 3"])
def test_bf16_output_alignment(env, case):
    # The bf16 epilogue stores 16-byte row pieces when the output's rows allow
    # it, else element by element: every placement gives the RNE of the same
    # call's fp32 output, and nothing outside the logical output is written.
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(23)
    M, K = 300, 336
    N = 203 if case == "N % 8 == 3" else 208
    x = wl.student_t_unit_var(rng, (M, K), 4)
    w = wl.normal(rng, (N, K), 0.02)
    print(f"bf16 output placement: {case}", flush=True)
    gx = q.nvfp4_quantize(to_dev(x, dev), layout=q.LAYOUT_INTERLEAVED)
    gw = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_1X16, q.RNE, layout=q.LAYOUT_INTERLEAVED)
    y32 = q.nvfp4_gemm(q.FPROP, gx, gw, torch.float32)
    ld = {"ldc % 8 == 4": N + 4, "8-byte aligned view": N + 24, "N % 8 == 3": 216}[case]
    assert ld % 4 == 0
    off = 4 if case == "8-byte aligned view" else 0
    buf = torch.full((M, ld + off), -3.0, dtype=torch.bfloat16, device=dev)
    out = buf[:, off:off + N]
    assert out.data_ptr() % 16 == (8 if off else 0)
    q.nvfp4_gemm(q.FPROP, gx, gw, out=out)
    torch.cuda.synchronize()
    assert (buf[:, :off] == -3.0).all().item() and (buf[:, off + N:] == -3.0).all().item()
    b16 = out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(b16, bf16_rne_bits(y32.cpu().numpy()))
    want = oracle.gemm(oracle.FPROP, oracle.quantize(x), oracle.quantize(w))
    assert rel_fro(y32.cpu().numpy(), want) <= TOL


def _scaled(wl, bits, f):
    return wl.f32_to_bf16_bits((wl.bf16_bits_to_f32(bits).astype(np.float64) * f).astype(np.float32))


# Extreme tensor scales (two-level scaling edges): (a factor, b factor).
# 1e-17 / 2e-18: the product of the FP32 decode scales falls below fp32's
# normal range while every output is normal; 1e-36: the tensor scale of A
# saturates at FLT_MAX (amax < 2688 / FLT_MAX); 0: A all zeros (s_enc = 1);
# 1e30 / 1e-30: a large and a small tensor scale.
EXTREME = {"both 1e-17": (1e-17, 1e-17 / 0.02), "both 2e-18": (2e-18, 2e-18 / 0.02),
           "a at FLT_MAX scale": (1e-36, 1.0 / 0.02), "a zero": (0.0, 1.0),
           "large and small": (1e30, 1e-30 / 0.02)}


@pytest.mark.parametrize("case", list(EXTREME))
@pytest.mark.parametrize("pass_name", ["fprop", "dgrad", "wgrad"])
def test_extreme_tensor_scales(env, case, pass_name):
    # Both datapaths within 1e-5 of the fp64 oracle (bf16 output = RNE of the
    # fp32 output), and the FP8-per-block datapath equal to the oracle's fp32
    # block GEMM bit for bit, at the edges of the tensor scale.
    torch, oracle, q, wl, dev = env
    fa, fb = EXTREME[case]
    M, K, N = 96, 272, 80
    rng = np.random.default_rng(123)
    print(f"extreme scales {case} {pass_name}", flush=True)
    if pass_name == "fprop":
        a = _scaled(wl, wl.normal(rng, (M, K), 1.0), fa)
        w = _scaled(wl, wl.normal(rng, (N, K), 0.02), fb)
        ga, gb = q.nvfp4_quantize(to_dev(a, dev)), q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, with_transpose=True)
        oa, ob = oracle.quantize(a), oracle.quantize(w, oracle.BLOCK_16X16)
        want, ob_rows, pass_ = oracle.gemm(oracle.FPROP, oa, ob), ob, q.FPROP
    elif pass_name == "dgrad":
        a = _scaled(wl, wl.lognormal_rows(rng, (M, N), base=1.0, sigma=0.5), fa)
        w = _scaled(wl, wl.normal(rng, (N, K), 0.02), fb)
        ga = q.nvfp4_quantize(to_dev(a, dev), q.BLOCK_1X16, q.SR, 7)
        gb = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, with_transpose=True)
        oa, ob = oracle.quantize(a, oracle.BLOCK_1X16, oracle.SR, 7), oracle.quantize(w, oracle.BLOCK_16X16)
        want, pass_ = oracle.gemm(oracle.DGRAD, oa, ob), q.DGRAD
        ob_rows = oracle.quantize(np.ascontiguousarray(w.T), oracle.BLOCK_16X16)
    else:
        dy = _scaled(wl, wl.lognormal_rows(rng, (K, M), base=1.0, sigma=0.5), fa)
        x = _scaled(wl, wl.normal(rng, (K, N), 0.02), fb)
        mask = q.nvfp4_rht_sign_mask(K)
        ga, gb = q.nvfp4_rht_quantize(to_dev(dy, dev), mask, q.SR, 9), q.nvfp4_rht_quantize(to_dev(x, dev), mask)
        oa, ob = oracle.rht_quantize(dy, mask, oracle.SR, 9), oracle.rht_quantize(x, mask)
        want, ob_rows, pass_ = oracle.gemm(oracle.WGRAD, oa, ob), ob, q.WGRAD
    if fa == 1e-36:
        assert np.float32(oa.s_enc) == np.finfo(np.float32).max  # the clamp is exercised
    if fa != 0.0:  # most outputs are normal fp32 numbers (cancellation may leave a few tiny)
        assert np.median(np.abs(want)) > 1e-36
    _check_both_dtypes(torch, q, pass_, ga, gb, want)
    y = q.nvfp4_gemm(pass_, ga, gb, torch.float32, fp8_blocks=True)
    torch.cuda.synchronize()
    got, ref = y.cpu().numpy(), oracle.gemm_fp32_blocks(oa, ob_rows)
    bad = np.argwhere(got.view(np.uint32) != ref.view(np.uint32))
    assert len(bad) == 0, f"{len(bad)} outputs differ, first {bad[0]}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
