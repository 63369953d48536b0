"""Parity of the sized RHT quantiser (nvfp4_rht_quantize_sized: 1, 4, 16
or 64-token transforms, the size ablation of "Pretraining Large Language
Models with NVFP4", Technische Zusammenfassung 2.B.2) with the oracle, bit
for bit, at sizes spanning several tiles with ragged channel tails, and for
the 12B-layer activation X in full."""
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


@pytest.mark.parametrize("size", [1, 4, 16, 64])
@pytest.mark.parametrize("shape", [(64, 8), (128, 24), (320, 200), (512, 264), (4096, 64)])
@pytest.mark.parametrize("rounding", [0, 1])
def test_sized_matches_oracle(env, size, shape, rounding):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(size * 1000 + shape[0] + shape[1] + rounding)
    x = wl.lognormal_rows(rng, shape) if rounding else wl.normal_with_outliers(rng, shape)
    signs = q.nvfp4_rht_signs64(int(rng.integers(0, 2 ** 32)))
    print(f"rht sized {size} {shape} r={rounding}", flush=True)
    g = q.nvfp4_rht_quantize_sized(to_dev(x, dev), size, signs, rounding, 31)
    torch.cuda.synchronize()
    assert_same_quant(g, oracle.rht_quantize_sized(x, size, signs, rounding, 31),
                      f"rht{size} {shape}")


def test_size16_equals_rht_quantize_and_amax_in(env):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(77)
    full = wl.student_t_unit_var(rng, (512, 160), 4)
    xd = to_dev(full, dev)[:, :136]                     # strided input
    x = np.ascontiguousarray(full[:, :136])
    signs = q.nvfp4_rht_signs64(5)
    print("rht sized 16 vs rht_quantize", flush=True)
    a = q.nvfp4_rht_quantize_sized(xd, 16, signs, q.SR, 4)
    b = q.nvfp4_rht_quantize(xd, signs & 0xFFFF, q.SR, 4)
    amax = torch.tensor([2.5], dtype=torch.float32, device=dev)
    c = q.nvfp4_rht_quantize_sized(xd, 64, signs, q.RNE, 0, amax_in=amax)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    assert a.amax.item() == b.amax.item()
    assert_same_quant(c, oracle.rht_quantize_sized(x, 64, signs, oracle.RNE, 0, amax_in=2.5),
                      "rht64 amax_in")


def test_sized_errors(env):
    torch, oracle, q, wl, dev = env
    x = torch.zeros((96, 16), dtype=torch.bfloat16, device=dev)
    with pytest.raises(RuntimeError, match="status -2"):
        q.nvfp4_rht_quantize_sized(x, 64, 0)            # 96 tokens: not whole 64-token chunks
    with pytest.raises(RuntimeError, match="status -4"):
        q.nvfp4_rht_quantize_sized(x, 8, 0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("size", [4, 64])
def test_sized_full_size(env, size):
    # the 12B-layer activation X (8192 tokens x 5120 channels), RNE
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(90 + size)
    x = wl.student_t_unit_var(rng, (8192, 5120), 3)
    signs = oracle.rht_signs64(1000)
    print(f"rht sized {size} full X", flush=True)
    g = q.nvfp4_rht_quantize_sized(to_dev(x, dev), size, signs, q.RNE)
    torch.cuda.synchronize()
    assert_same_quant(g, oracle.rht_quantize_sized(x, size, signs, oracle.RNE), f"rht{size} full X")


# --- RHT along the rows (fprop / dgrad operands) ------------------------------

@pytest.mark.parametrize("block", [0, 1])
@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (160, 1040), (272, 2064)])
@pytest.mark.parametrize("rounding", [0, 1])
def test_row_rht_matches_oracle(env, block, shape, rounding):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(block * 7 + shape[0] + shape[1] + rounding)
    x = wl.normal_with_outliers(rng, shape) if rounding == 0 else wl.lognormal_rows(rng, shape)
    mask = int(rng.integers(0, 65536))
    print(f"row rht block={block} {shape} r={rounding}", flush=True)
    g = q.nvfp4_quantize_rht_rows(to_dev(x, dev), mask, block, rounding, 17)
    torch.cuda.synchronize()
    assert_same_quant(g, oracle.quantize_rht_rows(x, mask, block, rounding, 17), f"row rht {shape}")


def test_row_rht_strided_amax_in_and_product(env):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(5)
    full = wl.student_t_unit_var(rng, (64, 336), 4)
    x = np.ascontiguousarray(full[:, :320])
    xd = to_dev(full, dev)[:, :320]
    print("row rht strided", flush=True)
    g = q.nvfp4_quantize_rht_rows(xd, 0x3C5A, 0, 1, 6)
    amax = torch.tensor([4.0], dtype=torch.float32, device=dev)
    h = q.nvfp4_quantize_rht_rows(xd, 0x3C5A, 1, 0, 0, amax_in=amax)
    torch.cuda.synchronize()
    assert_same_quant(g, oracle.quantize_rht_rows(x, 0x3C5A, 0, 1, 6), "row rht strided")
    assert_same_quant(h, oracle.quantize_rht_rows(x, 0x3C5A, 1, 0, 0, amax_in=4.0), "row rht amax_in")
    # the fprop GEMM on row-transformed operands approximates the plain product
    w = wl.normal(rng, (48, 320), 0.05)
    gw = q.nvfp4_quantize_rht_rows(to_dev(w, dev), 0x3C5A, 1, 0)
    gx = q.nvfp4_quantize_rht_rows(xd, 0x3C5A, 0, 0)
    y = q.nvfp4_gemm(q.FPROP, gx, gw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.gemm(oracle.FPROP, oracle.quantize_rht_rows(x, 0x3C5A, 0, 0),
                      oracle.quantize_rht_rows(w, 0x3C5A, 1, 0))
    from tests.gpu_util import rel_fro
    assert rel_fro(y.cpu().numpy(), ref) <= 1e-5
