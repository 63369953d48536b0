"""Parity of the dual quantiser (nvfp4_quantize_dual): one read of a tensor
gives its 1x16 operand and its RHT-transposed operand, each bit-identical to
the oracle's quantize() and rht_quantize() of the same tensor.

Sizes span several 256-token x 128-channel tiles with ragged tails in both
dimensions; the full-size cases are the 12B-layer gradient dY (8192 x 20480,
SR) and activation X (8192 x 5120, RNE), compared in full."""
import numpy as np
import pytest

from tests.gpu_util import assert_same_quant, ensure_built, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    ensure_built()
    import oracle
    import quantize_precision_gemm_amd as q
    from quantize_precision_gemm_amd import workloads as wl
    return torch, oracle, q, wl, torch.device("cuda:0")


def _check(env, x, mask, rounding, seed, seed_rht, what, xd=None, amax=None):
    torch, oracle, q, wl, dev = env
    xd = to_dev(x, dev) if xd is None else xd
    print(f"dual {what}", flush=True)
    if amax is None:
        g, gr = q.nvfp4_quantize_dual(xd, mask, rounding, seed, seed_rht)
        a = ar = None
    else:
        a, ar = amax
        g, gr = q.nvfp4_quantize_dual(xd, mask, rounding, seed, seed_rht,
                                      amax_in=torch.tensor([a], dtype=torch.float32, device=dev),
                                      amax_rht_in=torch.tensor([ar], dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    assert (g.rows, g.cols, gr.rows, gr.cols) == (x.shape[0], x.shape[1], x.shape[1], x.shape[0])
    assert_same_quant(g, oracle.quantize(x, oracle.BLOCK_1X16, rounding, seed, amax_in=a),
                      f"{what} 1x16")
    assert_same_quant(gr, oracle.rht_quantize(x, mask, rounding, seed_rht, amax_in=ar),
                      f"{what} rht")
    return g, gr


@pytest.mark.parametrize("shape", [(16, 16), (48, 32), (272, 208), (512, 272), (4096, 64),
                                   (304, 1040), (768, 384)])
@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("kind", ["normal", "rows"])
def test_dual_matches_oracle(env, shape, rounding, kind):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(shape[0] * 31 + shape[1] * 7 + rounding)
    x = wl.normal(rng, shape, 1.0) if kind == "normal" else wl.lognormal_rows(rng, shape)
    mask = int(rng.integers(0, 65536))
    _check(env, x, mask, rounding, int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 63)),
           f"{shape} r={rounding} {kind}")


def test_dual_same_as_separate_calls(env):
    # the fused pass and the two quantisers it replaces agree bit for bit,
    # with the maxima computed internally or passed in
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(5)
    xd = to_dev(wl.student_t_unit_var(rng, (1024, 640), 4), dev)
    print("dual vs separate", flush=True)
    a, ar = q.nvfp4_amax(xd, 0x5A5A)
    g, gr = q.nvfp4_quantize_dual(xd, 0x5A5A, q.SR, 11, 12)
    h, hr = q.nvfp4_quantize_dual(xd, 0x5A5A, q.SR, 11, 12, amax_in=a, amax_rht_in=ar)
    s = q.nvfp4_quantize(xd, q.BLOCK_1X16, q.SR, 11)
    sr = q.nvfp4_rht_quantize(xd, 0x5A5A, q.SR, 12)
    torch.cuda.synchronize()
    for u in (g, h):
        assert torch.equal(u.codes, s.codes) and torch.equal(u.scales, s.scales)
        assert u.amax.item() == s.amax.item() and u.s_enc.item() == s.s_enc.item()
    for u in (gr, hr):
        assert torch.equal(u.codes, sr.codes) and torch.equal(u.scales, sr.scales)
        assert u.amax.item() == sr.amax.item() and u.s_enc.item() == sr.s_enc.item()


def test_dual_strided_and_amax_in(env):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(9)
    full = wl.normal(rng, (272, 400), 1.0)
    x = np.ascontiguousarray(full[:, :336])
    xd = to_dev(full, dev)[:, :336]
    _check(env, x, 0x1357, 1, 3, 4, "strided", xd=xd)
    _check(env, x, 0x1357, 0, 0, 0, "strided amax_in", xd=xd, amax=(5.0, 7.5))


def test_dual_edge_tensors(env):
    torch, oracle, q, wl, dev = env
    zeros = np.zeros((32, 64), np.uint16)
    z = np.zeros((16, 32), np.uint16)
    z[2, 3] = 0x8000
    z[5, 17] = 0x0001                      # smallest bf16 subnormal
    big = np.zeros((16, 32), np.float32)
    big[0, 0] = 3.0e38
    big[1, 5:20] = -1.0
    tiny = (np.random.default_rng(1).standard_normal((32, 48)) * 1e-38).astype(np.float32)
    for name, x in [("zeros", zeros), ("neg_zero_subnormal", z),
                    ("huge", wl.f32_to_bf16_bits(big)), ("tiny", wl.f32_to_bf16_bits(tiny))]:
        for rounding in (0, 1):
            _check(env, x, 0xBEEF, rounding, 3, 4, f"edge {name} r={rounding}")


def test_dual_empty(env):
    torch, oracle, q, wl, dev = env
    print("dual empty", flush=True)
    for shape in [(0, 32), (32, 0)]:
        x = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        g, gr = q.nvfp4_quantize_dual(x, 1, q.SR, 1, 2)
        torch.cuda.synchronize()
        for t in (g, gr):
            assert t.amax.item() == 0.0 and t.s_enc.item() == 1.0
        assert (gr.rows, gr.cols) == (shape[1], shape[0])


def test_dual_errors(env):
    torch, oracle, q, wl, dev = env
    x = torch.zeros((32, 48), dtype=torch.bfloat16, device=dev)
    with pytest.raises(RuntimeError, match="status -2"):
        q.nvfp4_quantize_dual(x[:, :40], 1)          # channels not a multiple of 16
    with pytest.raises(RuntimeError, match="status -2"):
        q.nvfp4_quantize_dual(x[:24], 1)             # tokens not a multiple of 16
    with pytest.raises(RuntimeError, match="status -1"):
        q.nvfp4_quantize_dual(x, 1, amax_in=torch.ones(1, device=dev))
    torch.cuda.synchronize()


@pytest.mark.parametrize("what,shape,rounding", [("dY", (8192, 20480), 1), ("X", (8192, 5120), 0)])
def test_dual_full_size(env, what, shape, rounding):
    # the 12B-layer tensors in the launch configuration the step uses; the
    # oracle quantises the whole tensor both ways
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(21 if what == "dY" else 22)
    x = wl.normal(rng, shape, 1e-3 if what == "dY" else 1.0)
    mask = oracle.rht_sign_mask(1000)
    _check(env, x, mask, rounding, 100, 101, f"full {what} {shape}")


def test_step_schedules_agree(env):
    # a training step with the dual quantisers produces the same operands and
    # the same fprop / dgrad / wgrad outputs, bit for bit, as with separate ones
    torch, oracle, q, wl, dev = env
    from quantize_precision_gemm_amd.step import NVFP4Linear, TrainingStep
    rng = np.random.default_rng(17)
    M, K, N = 512, 384, 640
    x = to_dev(wl.normal(rng, (M, K), 1.0), dev)
    w = to_dev(wl.normal(rng, (N, K), 0.02), dev)
    dy = to_dev(wl.normal(rng, (M, N), 1e-3), dev)
    print("step schedules", flush=True)
    steps = [TrainingStep(torch, [NVFP4Linear(q, torch, x, w, dy, 7, fused)], dev)
             for fused in (False, True)]
    for s in steps:
        s.run()
    torch.cuda.synchronize()
    a, b = steps[0].layers[0], steps[1].layers[0]
    for name in ("gx", "gdy", "gdyt", "gxt"):
        ta, tb = getattr(a, name), getattr(b, name)
        assert np.array_equal(ta.codes_host(), tb.codes_host()), name
        assert torch.equal(ta.scales, tb.scales), name
        assert ta.s_enc.item() == tb.s_enc.item(), name
    for name in ("y", "dx", "dw"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
