"""GPU parity of the quantisers against the CPU oracle: codes, scales, amax and
s_enc bit-exact.

Recipe: "Pretraining Large Language Models with NVFP4" (gist.science
summary), Technische Zusammenfassung 2.A (format), 2.B.2 (RHT on wgrad
inputs), 2.B.3 (16x16 weight blocks), 2.B.4 (SR for gradients, RNE otherwise).
"""
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
    dev = torch.device("cuda:0")
    return torch, oracle, q, wl, dev


def _bits(wl, rng, shape, kind):
    if kind == "normal":
        return wl.normal(rng, shape, 1.0)
    if kind == "t4":
        return wl.student_t_unit_var(rng, shape, 4)
    if kind == "rows":
        return wl.lognormal_rows(rng, shape)
    if kind == "wide":
        x = rng.standard_normal(shape) * np.exp(rng.uniform(-40, 40, shape))
        return wl.f32_to_bf16_bits(x.astype(np.float32))
    if kind == "outliers":
        return wl.normal_with_outliers(rng, shape)
    raise ValueError(kind)


SHAPES_1X16 = [(1, 16), (3, 48), (37, 336), (256, 256), (300, 1040), (129, 4112)]


@pytest.mark.parametrize("shape", SHAPES_1X16)
@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("kind", ["normal", "rows", "wide"])
def test_quant_1x16(env, shape, rounding, kind):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(hash((shape, rounding, kind)) % 2 ** 32)
    x = _bits(wl, rng, shape, kind)
    seed = int(rng.integers(0, 2 ** 63))
    print(f"1x16 shape={shape} rounding={rounding} kind={kind}", flush=True)
    g = q.nvfp4_quantize(to_dev(x, dev), q.BLOCK_1X16, rounding, seed)
    torch.cuda.synchronize()
    assert_same_quant(g, oracle.quantize(x, oracle.BLOCK_1X16, rounding, seed), f"1x16 {shape}")


@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (64, 1056), (160, 2064)])
@pytest.mark.parametrize("rounding", [0, 1])
def test_quant_16x16_with_transpose(env, shape, rounding):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(sum(shape) + rounding)
    x = _bits(wl, rng, shape, "t4")
    seed = 12345
    print(f"16x16 shape={shape} rounding={rounding}", flush=True)
    g = q.nvfp4_quantize(to_dev(x, dev), q.BLOCK_16X16, rounding, seed, with_transpose=True)
    torch.cuda.synchronize()
    o = oracle.quantize(x, oracle.BLOCK_16X16, rounding, seed)
    ot = None
    if rounding == 0:  # SR draws are indexed in W's layout, so only RNE transposes exactly
        ot = oracle.quantize(np.ascontiguousarray(x.T), oracle.BLOCK_16X16, rounding, seed)
    assert_same_quant(g, o, f"16x16 {shape}", transposed=ot)
    if rounding == 1:
        codes = oracle.unpack_codes(o.codes, shape[1])
        gt = oracle.unpack_codes(g.codes_t_host(), shape[0])
        np.testing.assert_array_equal(gt, codes.T)
        np.testing.assert_array_equal(g.scales_t_host(), o.scales.T)


@pytest.mark.parametrize("shape", [(16, 8), (48, 24), (272, 200), (512, 264), (4096, 64)])
@pytest.mark.parametrize("rounding", [0, 1])
def test_rht_quant(env, shape, rounding):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(7 * shape[0] + shape[1] + rounding)
    x = _bits(wl, rng, shape, "rows" if rounding else "t4")
    mask = int(rng.integers(0, 65536))
    seed = 99
    print(f"rht shape={shape} rounding={rounding}", flush=True)
    g = q.nvfp4_rht_quantize(to_dev(x, dev), mask, rounding, seed)
    torch.cuda.synchronize()
    assert_same_quant(g, oracle.rht_quantize(x, mask, rounding, seed), f"rht {shape}")


def test_strided_input_and_amax_in(env):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(3)
    full = wl.normal(rng, (64, 96), 1.0)
    x = np.ascontiguousarray(full[:, :64])
    xd = to_dev(full, dev)[:, :64]
    print("strided", flush=True)
    g = q.nvfp4_quantize(xd, q.BLOCK_1X16, q.RNE)
    torch.cuda.synchronize()
    assert_same_quant(g, oracle.quantize(x), "strided 1x16")
    g2 = q.nvfp4_quantize(xd, q.BLOCK_16X16, q.RNE, with_transpose=True)
    torch.cuda.synchronize()
    assert_same_quant(g2, oracle.quantize(x, oracle.BLOCK_16X16), "strided 16x16")
    gr = q.nvfp4_rht_quantize(xd, 0x1234, q.SR, 5)
    torch.cuda.synchronize()
    assert_same_quant(gr, oracle.rht_quantize(x, 0x1234, oracle.SR, 5), "strided rht")
    amax = torch.tensor([3.5], dtype=torch.float32, device=dev)
    g3 = q.nvfp4_quantize(xd, q.BLOCK_1X16, q.SR, 8, amax_in=amax)
    torch.cuda.synchronize()
    assert_same_quant(g3, oracle.quantize(x, oracle.BLOCK_1X16, oracle.SR, 8, amax_in=3.5), "amax_in")


def _adversarial_rows(wl):
    """Blocks whose per-element factor is exactly 1 and whose elements cover every
    bf16 value in [0, 6.5] of both signs (all E2M1 ties), plus blocks whose scale
    computation lands on E4M3 ties; the tensor amax 2688 gives s_enc = 1."""
    vals = (np.arange(0, 1 << 16, dtype=np.uint32) << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 6.5)]
    pad = (-len(vals)) % 15
    vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, 15)
    blocks = np.concatenate([np.full((len(vals), 1), 6.0, np.float32), vals], axis=1)
    # E4M3 tie cases: amax_b / 6 on every midpoint between E4M3 values
    e4 = []
    for b in range(1, 0x7E):
        e, m = b >> 3, b & 7
        e4.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    e4 = np.array(e4)
    mids = (e4[1:] + e4[:-1]) / 2 * 6
    tie_blocks = np.zeros((len(mids), 16), np.float32)
    tie_blocks[:, 0] = mids
    tie_blocks[:, 1:] = mids[:, None] * np.linspace(-1, 1, 15)[None, :]
    x = np.concatenate([blocks, tie_blocks]).reshape(-1)
    x = np.concatenate([x, np.zeros((-len(x)) % 64, np.float32)]).reshape(-1, 64)
    x[0, 0] = 2688.0
    return wl.f32_to_bf16_bits(x)


@pytest.mark.parametrize("rounding", [0, 1])
def test_adversarial_ties(env, rounding):
    torch, oracle, q, wl, dev = env
    x = _adversarial_rows(wl)
    print(f"adversarial shape={x.shape}", flush=True)
    g = q.nvfp4_quantize(to_dev(x, dev), q.BLOCK_1X16, rounding, 77)
    torch.cuda.synchronize()
    o = oracle.quantize(x, oracle.BLOCK_1X16, rounding, 77)
    assert o.s_enc == 1.0
    assert_same_quant(g, o, "adversarial")


def test_edge_tensors(env):
    torch, oracle, q, wl, dev = env
    cases = {}
    cases["zeros"] = np.zeros((32, 64), np.uint16)
    z = np.zeros((16, 32), np.uint16)
    z[2, 3] = 0x8000
    z[5, 17] = 0x0001  # smallest bf16 subnormal
    cases["neg_zero_subnormal"] = z
    tiny = wl.f32_to_bf16_bits((np.random.default_rng(1).standard_normal((16, 48)) * 1e-38).astype(np.float32))
    cases["tiny_amax"] = tiny
    big = np.zeros((16, 32), np.float32)
    big[0, 0] = 3.0e38
    big[1, 5:20] = -1.0
    cases["huge"] = wl.f32_to_bf16_bits(big)
    under = np.zeros((16, 32), np.float32)
    under[0, 0] = 1e4
    under[3, 16:] = np.linspace(-1e-5, 1e-5, 16)
    cases["underflow_block"] = wl.f32_to_bf16_bits(under)
    for name, x in cases.items():
        for rounding in (0, 1):
            for block in (0, 1):
                print(f"edge {name} rounding={rounding} block={block}", flush=True)
                g = q.nvfp4_quantize(to_dev(x, dev), block, rounding, 3, with_transpose=block == 1)
                torch.cuda.synchronize()
                assert_same_quant(g, oracle.quantize(x, block, rounding, 3), f"{name}")
            if x.shape[0] % 16 == 0 and x.shape[1] % 8 == 0:
                gr = q.nvfp4_rht_quantize(to_dev(x, dev), 0xBEEF, rounding, 3)
                torch.cuda.synchronize()
                assert_same_quant(gr, oracle.rht_quantize(x, 0xBEEF, rounding, 3), f"rht {name}")


def test_empty(env):
    torch, oracle, q, wl, dev = env
    print("empty", flush=True)
    x = torch.empty((0, 32), dtype=torch.bfloat16, device=dev)
    g = q.nvfp4_quantize(x, q.BLOCK_1X16, q.RNE)
    torch.cuda.synchronize()
    assert g.amax.item() == 0.0 and g.s_enc.item() == 1.0
    x = torch.empty((32, 0), dtype=torch.bfloat16, device=dev)
    g = q.nvfp4_rht_quantize(torch.empty((0, 16), dtype=torch.bfloat16, device=dev), 1, q.RNE)
    torch.cuda.synchronize()
    assert g.amax.item() == 0.0 and g.s_enc.item() == 1.0


def test_determinism(env):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(11)
    x = to_dev(wl.lognormal_rows(rng, (512, 2048)), dev)
    print("determinism", flush=True)
    a = q.nvfp4_quantize(x, q.BLOCK_1X16, q.SR, 5)
    b = q.nvfp4_quantize(x, q.BLOCK_1X16, q.SR, 5)
    c = q.nvfp4_rht_quantize(x, 77, q.SR, 5)
    d = q.nvfp4_rht_quantize(x, 77, q.SR, 5)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    assert torch.equal(c.codes, d.codes) and torch.equal(c.scales, d.scales)
    e = q.nvfp4_quantize(x, q.BLOCK_1X16, q.SR, 6)
    torch.cuda.synchronize()
    assert not torch.equal(a.codes, e.codes)  # another seed draws other bits


def test_error_paths(env):
    torch, oracle, q, wl, dev = env
    x = torch.zeros((32, 48), dtype=torch.bfloat16, device=dev)
    with pytest.raises(RuntimeError, match="status -2"):
        q.nvfp4_quantize(x[:, :40], q.BLOCK_1X16, q.RNE)      # cols not a multiple of 16
    with pytest.raises(RuntimeError, match="status -2"):
        q.nvfp4_quantize(x[:24], q.BLOCK_16X16, q.RNE)        # rows not a multiple of 16
    with pytest.raises(RuntimeError, match="status -4"):
        q.nvfp4_quantize(x, 7, q.RNE)
    with pytest.raises(RuntimeError, match="status -4"):
        q.nvfp4_quantize(x, q.BLOCK_1X16, 9)
    with pytest.raises(RuntimeError, match="status -3"):
        q.nvfp4_quantize(x[:, 1:33], q.BLOCK_1X16, q.RNE)     # misaligned start
    with pytest.raises(RuntimeError, match="status -2"):
        q.nvfp4_rht_quantize(x[:24], 1, q.RNE)                # tokens not a multiple of 16
    a = q.nvfp4_quantize(x, q.BLOCK_1X16, q.RNE)
    w = q.nvfp4_quantize(torch.zeros((16, 32), dtype=torch.bfloat16, device=dev), q.BLOCK_16X16, q.RNE)
    with pytest.raises(RuntimeError, match="status -5"):
        q.nvfp4_gemm(q.FPROP, a, w)                           # K mismatch 48 vs 32
    with pytest.raises(ValueError, match="transposed copy"):
        q.nvfp4_gemm(q.DGRAD, a, w)                           # no transposed copy: the binding
    import ctypes                                             # ... and the C ABI (-1) refuse it
    c = torch.empty((32, 32), dtype=torch.bfloat16, device=dev)
    da, dw = a.descriptor(), w.descriptor()
    st = q.load_library().nvfp4_gemm(q.DGRAD, ctypes.byref(da), ctypes.byref(dw), c.data_ptr(), 32,
                                     q.OUT_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == -1
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [(16, 8), (272, 200), (512, 264), (48, 1040)])
def test_fused_amax_matches_quantisers(env, shape):
    # one pass gives max |x| and max |RHT(x)|; fed back as amax_in the
    # quantisers produce exactly the oracle's codes and scales
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(shape[0] * 3 + shape[1])
    x = wl.lognormal_rows(rng, shape)
    mask = int(rng.integers(0, 65536))
    xd = to_dev(x, dev)
    print(f"fused amax {shape}", flush=True)
    a, ar = q.nvfp4_amax(xd, mask)
    a_only, none = q.nvfp4_amax(xd)
    torch.cuda.synchronize()
    assert none is None
    o1 = oracle.quantize(x, oracle.BLOCK_1X16, oracle.SR, 4) if shape[1] % 16 == 0 else None
    orht = oracle.rht_quantize(x, mask, oracle.SR, 5)
    assert np.float32(ar.item()) == np.float32(orht.amax)
    assert np.float32(a.item()) == np.float32(a_only.item())
    assert np.float32(a.item()) == np.float32(np.abs(wl.bf16_bits_to_f32(x)).max())
    g = q.nvfp4_rht_quantize(xd, mask, q.SR, 5, amax_in=ar)
    torch.cuda.synchronize()
    assert_same_quant(g, orht, f"rht with fused amax {shape}")
    if o1 is not None:
        g1 = q.nvfp4_quantize(xd, q.BLOCK_1X16, q.SR, 4, amax_in=a)
        torch.cuda.synchronize()
        assert_same_quant(g1, o1, f"1x16 with fused amax {shape}")


def test_binding_rejects_undersized_buffers_before_launch(env):
    # A 16x16-block buffer (rows/16 scale rows) reused for a 1x16 quantise, a
    # GEMM output of the wrong shape: the binding raises and nothing is written.
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(90)
    x = to_dev(wl.normal(rng, (64, 96), 1.0), dev)
    print("binding buffer checks", flush=True)
    out2d = q.alloc_nvfp4(64, 96, q.BLOCK_16X16, False, dev)
    out2d.scales.fill_(0xAB)
    with pytest.raises(ValueError):
        q.nvfp4_quantize(x, q.BLOCK_1X16, q.RNE, out=out2d)
    torch.cuda.synchronize()
    assert (out2d.scales == 0xAB).all().item()
    gx = q.nvfp4_quantize(x)
    gw = q.nvfp4_quantize(to_dev(wl.normal(rng, (32, 96), 0.02), dev), q.BLOCK_16X16)
    bad = torch.full((64, 31), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        q.nvfp4_gemm(q.FPROP, gx, gw, out=bad)
    with pytest.raises(ValueError):  # dgrad needs the transposed weight copy
        q.nvfp4_gemm(q.DGRAD, q.nvfp4_quantize(to_dev(wl.normal(rng, (64, 32), 1.0), dev)), gw)
    torch.cuda.synchronize()
    assert (bad == 7.0).all().item()
