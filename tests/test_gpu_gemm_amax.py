"""Parity of the GEMM whose epilogue also emits the output's tensor maxima
(nvfp4_gemm_amax): the bf16 output equals nvfp4_gemm's bit for bit, amax
equals the oracle's max |c| and amax_rht the oracle's max |RHT(c)| over
16-token chunks, exactly; the dual quantiser run with those maxima equals
the oracle's quantisation of the output.

Passes: "Pretraining Large Language Models with NVFP4" (gist.science
summary), Technische Zusammenfassung 2.A (tensor scale from the amax) and
2.B.2 (the output feeds the next layer's fprop and wgrad operands).
Shapes span several 256 x 256 tiles with ragged tails; M = 272 and 400
end in a half 32-row group (a lone 16-token chunk)."""
import numpy as np
import pytest

from tests.gpu_util import assert_same_quant, ensure_built, rel_fro, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    ensure_built()
    import oracle
    import quantize_precision_gemm_amd as q
    from quantize_precision_gemm_amd import workloads as wl
    return torch, oracle, q, wl, torch.device("cuda:0")


def _operands(env, pass_name, M, K, N, rng, scale=1.0):
    """Device operands of one pass and the oracle's quantised ones.
    fprop: X (M x K), W (N x K) -> M x N; dgrad: dY (M x N), W (N x K) -> M x K."""
    torch, oracle, q, wl, dev = env
    w = wl.normal(rng, (N, K), 0.02)
    gw = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE, with_transpose=True)
    ow = oracle.quantize(w, oracle.BLOCK_16X16)
    if pass_name == "fprop":
        x = wl.student_t_unit_var(rng, (M, K), 4) if scale == 1.0 else wl.normal(rng, (M, K), scale)
        return q.FPROP, q.nvfp4_quantize(to_dev(x, dev)), gw, oracle.FPROP, oracle.quantize(x), ow
    dy = wl.lognormal_rows(rng, (M, N)) if scale == 1.0 else wl.normal(rng, (M, N), scale)
    return (q.DGRAD, q.nvfp4_quantize(to_dev(dy, dev), q.BLOCK_1X16, q.SR, 17), gw, oracle.DGRAD,
            oracle.quantize(dy, oracle.BLOCK_1X16, oracle.SR, 17), ow)


def _bits(torch, c):
    return c.view(torch.int16).cpu().numpy().view(np.uint16)


def _check_maxima(env, P, ga, gb, mask, what, rht=True):
    torch, oracle, q, wl, dev = env
    c, am, ar = q.nvfp4_gemm_amax(P, ga, gb, mask, rht=rht)
    ref = q.nvfp4_gemm(P, ga, gb, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), ref.view(torch.int16)), f"{what}: output"
    ch = _bits(torch, c)
    assert am.item() == oracle.amax(ch), f"{what}: amax"
    if rht:
        assert ar.item() == oracle.rht_amax(ch, mask), f"{what}: amax of the transform"
    else:
        assert ar is None
    return c, am, ar, ch


SHAPES = [(16, 48, 32), (272, 336, 208), (400, 1040, 528), (512, 512, 768), (48, 4112, 96)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("pass_name", ["fprop", "dgrad"])
def test_gemm_amax_matches_oracle(env, pass_name, shape):
    torch, oracle, q, wl, dev = env
    M, K, N = shape
    rng = np.random.default_rng(7 * M + K + 3 * N + (pass_name == "dgrad"))
    mask = int(rng.integers(0, 65536))
    print(f"gemm amax {pass_name} {shape}", flush=True)
    P, ga, gb, OP, oa, ob = _operands(env, pass_name, M, K, N, rng)
    c, am, ar, ch = _check_maxima(env, P, ga, gb, mask, f"{pass_name} {shape}")
    # the output is the product: within bf16 rounding of the oracle's
    want = oracle.gemm(OP, oa, ob)
    assert rel_fro(wl.bf16_bits_to_f32(ch).astype(np.float64), want) <= 2.0 ** -8
    # the next layer's operands from one read of c with the emitted maxima
    g, gr = q.nvfp4_quantize_dual(c, mask, q.SR, 5, 6, amax_in=am, amax_rht_in=ar)
    torch.cuda.synchronize()
    assert_same_quant(g, oracle.quantize(ch, oracle.BLOCK_1X16, oracle.SR, 5), f"{shape} 1x16")
    assert_same_quant(gr, oracle.rht_quantize(ch, mask, oracle.SR, 6), f"{shape} rht")


def test_gemm_amax_plain_only_and_reuse(env):
    # without the transform any row count works; a second call into the same
    # maxima buffers with a smaller output starts again from zero
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(31)
    print("gemm amax plain / reuse", flush=True)
    P, ga, gb, *_ = _operands(env, "fprop", 40, 160, 96, rng)
    _check_maxima(env, P, ga, gb, 0, "plain M=40", rht=False)
    P, ga, gb, *_ = _operands(env, "fprop", 288, 320, 272, rng)
    c, am, ar, _ = _check_maxima(env, P, ga, gb, 0x9A3C, "first")
    first = (am.item(), ar.item())
    P, ga, gb, *_ = _operands(env, "fprop", 64, 320, 80, rng, scale=1e-3)
    c2, am2, ar2 = q.nvfp4_gemm_amax(P, ga, gb, 0x9A3C, amax=am, amax_rht=ar)
    torch.cuda.synchronize()
    ch = _bits(torch, c2)
    assert am2.data_ptr() == am.data_ptr() and ar2.data_ptr() == ar.data_ptr()
    assert am.item() == oracle.amax(ch) and ar.item() == oracle.rht_amax(ch, 0x9A3C)
    assert am.item() < first[0] and ar.item() < first[1]


def test_gemm_amax_empty(env):
    torch, oracle, q, wl, dev = env
    print("gemm amax empty", flush=True)
    a = q.alloc_nvfp4(32, 0)
    b = q.alloc_nvfp4(48, 0, q.BLOCK_16X16)
    for t in (a, b):
        t.amax.fill_(0)
        t.s_enc.fill_(1)
    am = torch.full((1,), 7.0, device=dev)
    ar = torch.full((1,), 7.0, device=dev)
    c, _, _ = q.nvfp4_gemm_amax(q.FPROP, a, b, 1, amax=am, amax_rht=ar)
    torch.cuda.synchronize()
    assert (c.float() == 0).all() and am.item() == 0.0 and ar.item() == 0.0
    e = q.alloc_nvfp4(0, 64)
    e.s_enc.fill_(1)
    rng = np.random.default_rng(2)
    gw = q.nvfp4_quantize(to_dev(wl.normal(rng, (48, 64), 1.0), dev), q.BLOCK_16X16, q.RNE,
                          with_transpose=True)
    c, am, ar = q.nvfp4_gemm_amax(q.FPROP, e, gw, 1)
    torch.cuda.synchronize()
    assert c.shape == (0, 48) and am.item() == 0.0 and ar.item() == 0.0


def test_gemm_amax_errors(env):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(4)
    print("gemm amax errors", flush=True)
    P, ga, gb, *_ = _operands(env, "fprop", 40, 64, 32, rng)
    with pytest.raises(RuntimeError, match="status -2"):
        q.nvfp4_gemm_amax(P, ga, gb, 1)                  # 40 rows: not whole 16-token chunks
    x = q.nvfp4_quantize(to_dev(wl.normal(rng, (32, 64), 1.0), dev))
    with pytest.raises(RuntimeError, match="status -4"):
        q.nvfp4_gemm_amax(q.WGRAD, x, x, 1)              # wgrad's output is not re-quantised
    torch.cuda.synchronize()


@pytest.mark.parametrize("pass_name", ["fprop", "dgrad"])
def test_gemm_amax_full_size(env, pass_name):
    # the 12B-layer GEMMs (M = 8192 tokens, K = 5120, N = 20480) in the
    # launch configuration the benchmark times; the oracle reduces the whole
    # output
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(41 if pass_name == "fprop" else 42)
    M, K, N = 8192, 5120, 20480
    print(f"gemm amax full {pass_name}", flush=True)
    w = to_dev(wl.normal(rng, (N, K), 0.02), dev)
    gw = q.nvfp4_quantize(w, q.BLOCK_16X16, q.RNE, with_transpose=True)
    del w
    if pass_name == "fprop":
        ga = q.nvfp4_quantize(to_dev(wl.student_t_unit_var(rng, (M, K), 4), dev))
        P = q.FPROP
    else:
        ga = q.nvfp4_quantize(to_dev(wl.normal(rng, (M, N), 1e-3), dev), q.BLOCK_1X16, q.SR, 3)
        P = q.DGRAD
    _check_maxima(env, P, ga, gb=gw, mask=oracle.rht_sign_mask(77), what=f"full {pass_name}")
