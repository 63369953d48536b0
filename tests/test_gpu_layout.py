"""GPU checks of the interleaved code layout (nvfp4_tensor.layout =
NVFP4_LAYOUT_INTERLEAVED, include/nvfp4.h).

Quantisers: with an interleaved output every NVFP4 quantiser writes the
bytes of its row-major result at the offsets the header defines, evaluated
here on the host from the formula itself (not through the binding's
conversion), with the same scales and tensor scalars; one case per
quantiser is also compared with the oracle through the binding's read-back.
GEMMs: every NVFP4 GEMM entry point gives bit-identical outputs whether
each operand's codes are row-major or interleaved, in any mix, on ragged
M and N and K tails; the row-major results are the ones the other GPU
modules pin to the oracle, and one case per pass is checked against the
oracle here too.  Only the placement of bytes changes, so the bar is
bit-exact.  Format: "Pretraining Large Language Models with NVFP4"
(gist.science summary), Technische Zusammenfassung 2.A; passes 2.B.2.
"""
import numpy as np
import pytest

from tests.gpu_util import assert_same_quant, ensure_built, rel_fro, to_dev

pytestmark = pytest.mark.gpu

IL = 1  # NVFP4_LAYOUT_INTERLEAVED


@pytest.fixture(scope="module")
def env():
    import torch
    ensure_built()
    import oracle
    import quantize_precision_gemm_amd as q
    from quantize_precision_gemm_amd import workloads as wl
    dev = torch.device("cuda:0")
    return torch, oracle, q, wl, dev


def _offsets(rows, nbytes, ld):
    """Flat offsets of bytes (r, j), r < rows, j < nbytes, in an interleaved
    buffer with ld-byte rows: the header's formula."""
    r = np.arange(rows, dtype=np.int64)[:, None]
    j = np.arange(nbytes, dtype=np.int64)[None, :]
    return (r // 4) * 4 * ld + (j // 32) * 128 + (r % 4) * 32 + j % 32


def _raw_matches(buf, want):
    """The interleaved device buffer `buf` holds the row-major bytes `want`."""
    raw = buf.cpu().numpy()
    assert raw.shape[0] % 4 == 0 and raw.shape[0] >= want.shape[0]
    assert raw.shape[1] % 32 == 0
    got = raw.reshape(-1)[_offsets(want.shape[0], want.shape[1], raw.shape[1])]
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{len(bad)} code bytes misplaced, first at {tuple(bad[0])}")


def _same_result(torch, gi, gr, transposed=False):
    """Interleaved result gi against the row-major result gr of the same call."""
    assert gi.layout == IL
    assert torch.equal(gi.amax.view(torch.int32), gr.amax.view(torch.int32))
    assert torch.equal(gi.s_enc.view(torch.int32), gr.s_enc.view(torch.int32))
    _raw_matches(gi.codes, gr.codes_host())
    np.testing.assert_array_equal(gi.scales_host(), gr.scales_host())
    np.testing.assert_array_equal(gi.codes_host(), gr.codes_host())
    if transposed:
        _raw_matches(gi.codes_t, gr.codes_t_host())
        np.testing.assert_array_equal(gi.scales_t_host(), gr.scales_t_host())


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (37, 336), (300, 1040), (129, 4112)])
@pytest.mark.parametrize("rounding", [0, 1])
def test_quantize_1x16(env, shape, rounding):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(shape[0] * 7 + shape[1] + rounding)
    x = wl.lognormal_rows(rng, shape)
    print(f"layout 1x16 {shape} rounding={rounding}", flush=True)
    xd = to_dev(x, dev)
    gr = q.nvfp4_quantize(xd, q.BLOCK_1X16, rounding, 99)
    gi = q.nvfp4_quantize(xd, q.BLOCK_1X16, rounding, 99, layout=IL)
    torch.cuda.synchronize()
    _same_result(torch, gi, gr)
    if shape == (37, 336):
        assert_same_quant(gi, oracle.quantize(x, oracle.BLOCK_1X16, rounding, 99), "1x16 il")


@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (64, 1056), (160, 2064)])
@pytest.mark.parametrize("rounding", [0, 1])
def test_quantize_16x16_with_transpose(env, shape, rounding):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(shape[0] * 5 + shape[1] + rounding)
    w = wl.normal(rng, shape, 0.02)
    print(f"layout 16x16 {shape} rounding={rounding}", flush=True)
    wd = to_dev(w, dev)
    gr = q.nvfp4_quantize(wd, q.BLOCK_16X16, rounding, 5, with_transpose=True)
    gi = q.nvfp4_quantize(wd, q.BLOCK_16X16, rounding, 5, with_transpose=True, layout=IL)
    torch.cuda.synchronize()
    _same_result(torch, gi, gr, transposed=True)
    if shape == (48, 80) and rounding == 0:
        assert_same_quant(gi, oracle.quantize(w, oracle.BLOCK_16X16), "16x16 il",
                          transposed=oracle.quantize(np.ascontiguousarray(w.T), oracle.BLOCK_16X16))


def _logical(buf, rows, nbytes):
    """Row-major view (all buffer rows x ld) of an interleaved buffer, and a
    mask of the bytes outside the logical rows x nbytes."""
    raw = buf.cpu().numpy()
    full = raw.reshape(-1)[_offsets(raw.shape[0], raw.shape[1], raw.shape[1])]
    outside = np.ones(full.shape, bool)
    outside[:rows, :nbytes] = False
    return full, outside


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (37, 336), (300, 1040), (129, 4112), (64, 5120)])
@pytest.mark.parametrize("rounding", [0, 1])
def test_quantize_1x16_interleaved_against_oracle(env, shape, rounding):
    # The interleaved 1x16 encoder against the oracle: ragged 4-row groups
    # and 512-column chunks, magnitudes over 80 binades per block, and
    # nothing written outside the logical codes and scales.
    torch, oracle, q, wl, dev = env
    rows, cols = shape
    rng = np.random.default_rng(rows * 13 + cols + rounding)
    mag = np.exp(rng.uniform(-40, 40, (rows, cols // 16))).repeat(16, 1)
    w = wl.f32_to_bf16_bits((rng.standard_normal(shape) * mag).astype(np.float32))
    print(f"1x16 interleaved {shape} rounding={rounding}", flush=True)
    out = q.alloc_nvfp4(rows, cols, q.BLOCK_1X16, False, dev, IL)
    out.codes.fill_(0xAB)
    out.scales.fill_(0xAB)
    g = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_1X16, rounding, 77, out=out, layout=IL)
    torch.cuda.synchronize()
    assert_same_quant(g, oracle.quantize(w, oracle.BLOCK_1X16, rounding, 77), "1x16 il")
    full, outside = _logical(g.codes, rows, cols // 2)
    assert (full[outside] == 0xAB).all(), "codes written outside the tensor"
    sc = g.scales.cpu().numpy()
    assert (sc[:, cols // 16:] == 0xAB).all() and (sc[rows:] == 0xAB).all()


@pytest.mark.parametrize("shape", [(16, 16), (272, 208), (64, 1056), (160, 2064), (336, 528)])
@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("transpose", [True, False])
def test_quantize_16x16_interleaved_against_oracle(env, shape, rounding, transpose):
    # The interleaved 16x16 encoder against the oracle: ragged tile rows
    # (a workgroup takes 4) and column chunks (512 per wave), magnitudes over
    # 80 binades, and nothing written outside the logical codes and scales.
    torch, oracle, q, wl, dev = env
    rows, cols = shape
    rng = np.random.default_rng(rows * 3 + cols + 11 * rounding)
    tile_mag = np.exp(rng.uniform(-40, 40, (rows // 16, cols // 16)))
    x = rng.standard_normal(shape) * tile_mag.repeat(16, 0).repeat(16, 1)
    w = wl.f32_to_bf16_bits(x.astype(np.float32))
    print(f"16x16 interleaved {shape} rounding={rounding} transpose={transpose}", flush=True)
    out = q.alloc_nvfp4(rows, cols, q.BLOCK_16X16, transpose, dev, IL)
    for t in (out.codes, out.scales, out.codes_t, out.scales_t):
        if t is not None:
            t.fill_(0xAB)
    g = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, rounding, 31, with_transpose=transpose,
                         out=out, layout=IL)
    torch.cuda.synchronize()
    o = oracle.quantize(w, oracle.BLOCK_16X16, rounding, 31)
    assert_same_quant(g, o, "16x16 il")
    full, outside = _logical(g.codes, rows, cols // 2)
    assert (full[outside] == 0xAB).all(), "codes written outside the tensor"
    sc = g.scales.cpu().numpy()
    assert (sc[:, cols // 16:] == 0xAB).all() and (sc[rows // 16:] == 0xAB).all()
    if not transpose:
        return
    if rounding == 0:
        ot = oracle.quantize(np.ascontiguousarray(w.T), oracle.BLOCK_16X16)
        np.testing.assert_array_equal(g.codes_t_host(), ot.codes)
        np.testing.assert_array_equal(g.scales_t_host(), ot.scales)
    else:  # SR draws are indexed in W's layout: the copy is the same codes, transposed
        codes = oracle.unpack_codes(o.codes, cols)
        np.testing.assert_array_equal(oracle.unpack_codes(g.codes_t_host(), rows), codes.T)
        np.testing.assert_array_equal(g.scales_t_host(), o.scales.T)
    full, outside = _logical(g.codes_t, cols, rows // 2)
    assert (full[outside] == 0xAB).all(), "transposed codes written outside the tensor"
    st = g.scales_t.cpu().numpy()
    assert (st[:, rows // 16:] == 0xAB).all() and (st[cols // 16:] == 0xAB).all()


@pytest.mark.parametrize("shape", [(16, 8), (64, 72), (272, 264), (1040, 136)])
@pytest.mark.parametrize("rounding", [0, 1])
def test_rht_quantize(env, shape, rounding):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(shape[0] * 3 + shape[1] + rounding)
    x = wl.student_t_unit_var(rng, shape, 4)
    mask = q.nvfp4_rht_sign_mask(shape[0])
    print(f"layout rht {shape} rounding={rounding}", flush=True)
    xd = to_dev(x, dev)
    gr = q.nvfp4_rht_quantize(xd, mask, rounding, 13)
    gi = q.nvfp4_rht_quantize(xd, mask, rounding, 13, layout=IL)
    torch.cuda.synchronize()
    _same_result(torch, gi, gr)
    if shape == (272, 264):
        assert_same_quant(gi, oracle.rht_quantize(x, mask, rounding, 13), "rht il")


@pytest.mark.parametrize("shape", [(48, 80), (272, 208)])
@pytest.mark.parametrize("rounding", [0, 1])
def test_dual(env, shape, rounding):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(shape[0] + shape[1] * 11 + rounding)
    x = wl.lognormal_rows(rng, shape)
    mask = q.nvfp4_rht_sign_mask(3)
    print(f"layout dual {shape} rounding={rounding}", flush=True)
    xd = to_dev(x, dev)
    ar, br = q.nvfp4_quantize_dual(xd, mask, rounding, 1, 2)
    ai, bi = q.nvfp4_quantize_dual(xd, mask, rounding, 1, 2, layout=IL)
    # one result of each layout from one call
    am = q.alloc_nvfp4(shape[0], shape[1], q.BLOCK_1X16, device=dev)
    bm = q.alloc_nvfp4(shape[1], shape[0], q.BLOCK_1X16, device=dev, layout=IL)
    q.nvfp4_quantize_dual(xd, mask, rounding, 1, 2, out=am, out_rht=bm)
    torch.cuda.synchronize()
    _same_result(torch, ai, ar)
    _same_result(torch, bi, br)
    _same_result(torch, bm, br)
    np.testing.assert_array_equal(am.codes_host(), ar.codes_host())


@pytest.mark.parametrize("block", [0, 1])
def test_quantize_rht_rows(env, block):
    torch, oracle, q, wl, dev = env
    shape = (37, 336) if block == 0 else (48, 80)
    rng = np.random.default_rng(block + 77)
    x = wl.normal(rng, shape, 1.0)
    mask = q.nvfp4_rht_sign_mask(8)
    print(f"layout rht rows block={block}", flush=True)
    xd = to_dev(x, dev)
    wt = block == 1
    gr = q.nvfp4_quantize_rht_rows(xd, mask, block, q.RNE, with_transpose=wt)
    gi = q.nvfp4_quantize_rht_rows(xd, mask, block, q.RNE, with_transpose=wt, layout=IL)
    torch.cuda.synchronize()
    _same_result(torch, gi, gr, transposed=wt)


@pytest.mark.parametrize("size", [1, 4, 16, 64])
def test_rht_quantize_sized(env, size):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(size)
    x = wl.student_t_unit_var(rng, (192, 72), 4)
    signs = q.nvfp4_rht_signs64(size)
    print(f"layout rht sized {size}", flush=True)
    xd = to_dev(x, dev)
    gr = q.nvfp4_rht_quantize_sized(xd, size, signs, q.SR, 3)
    gi = q.nvfp4_rht_quantize_sized(xd, size, signs, q.SR, 3, layout=IL)
    torch.cuda.synchronize()
    _same_result(torch, gi, gr)


def _operands(q, wl, rng, dev, pass_name, M, K, N, layout_a, layout_b):
    if pass_name == "fprop":
        x = wl.student_t_unit_var(rng, (M, K), 4)
        w = wl.normal(rng, (N, K), 0.02)
        a = q.nvfp4_quantize(to_dev(x, dev), layout=layout_a)
        b = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE, with_transpose=True,
                             layout=layout_b)
        return q.FPROP, a, b
    if pass_name == "dgrad":
        dy = wl.lognormal_rows(rng, (M, N))
        w = wl.normal(rng, (N, K), 0.02)
        a = q.nvfp4_quantize(to_dev(dy, dev), q.BLOCK_1X16, q.SR, 3, layout=layout_a)
        b = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE, with_transpose=True,
                             layout=layout_b)
        return q.DGRAD, a, b
    Mt = (M + 15) // 16 * 16
    dy = wl.lognormal_rows(rng, (Mt, N))
    x = wl.student_t_unit_var(rng, (Mt, K), 4)
    mask = q.nvfp4_rht_sign_mask(Mt)
    a = q.nvfp4_rht_quantize(to_dev(dy, dev), mask, q.SR, 5, layout=layout_a)
    b = q.nvfp4_rht_quantize(to_dev(x, dev), mask, q.RNE, layout=layout_b)
    return q.WGRAD, a, b


def _all_outputs(torch, q, pass_, a, b):
    """Every NVFP4 GEMM entry point on (a, b), as int views for bitwise compares."""
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        iv = torch.int32 if dt == torch.float32 else torch.int16
        outs[f"gemm {dt}"] = q.nvfp4_gemm(pass_, a, b, dt).view(iv)
        outs[f"fp8blk {dt}"] = q.nvfp4_gemm(pass_, a, b, dt, fp8_blocks=True).view(iv)
        outs[f"split {dt}"] = q.nvfp4_gemm_split(pass_, a, b, None, dt).view(iv)
    if pass_ != q.WGRAD:
        rht = a.rows % 16 == 0  # the transform's maximum needs whole 16-row chunks
        c, am, amr = q.nvfp4_gemm_amax(pass_, a, b, sign_mask=0x5A5A, rht=rht)
        outs["amax gemm"] = c.view(torch.int16)
        outs["amax"] = am.view(torch.int32)
        if rht:
            outs["amax rht"] = amr.view(torch.int32)
    return outs


# (M, K, N): ragged M and N, K tails (K % 64 = 16), several 256-tiles, and
# shapes whose tiles leave a partial last wave (the split entry point splits it)
SHAPES = [(1, 16, 16), (300, 336, 272), (257, 1040, 528), (64, 4112, 96), (520, 512, 784)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("pass_name", ["fprop", "dgrad", "wgrad"])
def test_gemm_layouts_bitwise(env, pass_name, shape):
    torch, oracle, q, wl, dev = env
    M, K, N = shape
    print(f"layout gemm {pass_name} {shape}", flush=True)
    ref = None
    for la, lb in [(0, 0), (IL, IL), (IL, 0), (0, IL)]:
        rng = np.random.default_rng(13 * M + 7 * K + N)  # the same inputs for every layout
        pass_, a, b = _operands(q, wl, rng, dev, pass_name, M, K, N, la, lb)
        outs = _all_outputs(torch, q, pass_, a, b)
        torch.cuda.synchronize()
        if ref is None:
            ref = outs
            continue
        for k, v in outs.items():
            assert torch.equal(v, ref[k]), f"{k}: layouts ({la}, {lb}) differ from row-major"


@pytest.mark.parametrize("pass_name", ["fprop", "dgrad", "wgrad"])
def test_gemm_interleaved_against_oracle(env, pass_name):
    torch, oracle, q, wl, dev = env
    M, K, N = 300, 336, 272
    rng = np.random.default_rng(5)
    print(f"layout gemm oracle {pass_name}", flush=True)
    if pass_name == "fprop":
        x = wl.student_t_unit_var(rng, (M, K), 4)
        w = wl.normal(rng, (N, K), 0.02)
        a = q.nvfp4_quantize(to_dev(x, dev), layout=IL)
        b = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE, with_transpose=True, layout=IL)
        want = oracle.gemm(oracle.FPROP, oracle.quantize(x), oracle.quantize(w, oracle.BLOCK_16X16))
        pass_ = q.FPROP
    elif pass_name == "dgrad":
        dy = wl.lognormal_rows(rng, (M, N))
        w = wl.normal(rng, (N, K), 0.02)
        a = q.nvfp4_quantize(to_dev(dy, dev), q.BLOCK_1X16, q.SR, 17, layout=IL)
        b = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, q.RNE, with_transpose=True, layout=IL)
        want = oracle.gemm(oracle.DGRAD, oracle.quantize(dy, oracle.BLOCK_1X16, oracle.SR, 17),
                           oracle.quantize(w, oracle.BLOCK_16X16))
        pass_ = q.DGRAD
    else:
        Mt = 304
        dy = wl.lognormal_rows(rng, (Mt, N))
        x = wl.student_t_unit_var(rng, (Mt, K), 4)
        mask = q.nvfp4_rht_sign_mask(Mt)
        a = q.nvfp4_rht_quantize(to_dev(dy, dev), mask, q.SR, 23, layout=IL)
        b = q.nvfp4_rht_quantize(to_dev(x, dev), mask, q.RNE, layout=IL)
        want = oracle.gemm(oracle.WGRAD, oracle.rht_quantize(dy, mask, oracle.SR, 23),
                           oracle.rht_quantize(x, mask, oracle.RNE))
        pass_ = q.WGRAD
    y = q.nvfp4_gemm(pass_, a, b, torch.float32)
    torch.cuda.synchronize()
    err = rel_fro(y.cpu().numpy(), want)
    assert err <= 1e-5, f"relative Frobenius error {err:.3e}"


def test_binding_checks_interleaved_buffers(env):
    torch, oracle, q, wl, dev = env
    x = to_dev(wl.normal(np.random.default_rng(0), (6, 64), 1.0), dev)
    out = q.alloc_nvfp4(6, 64, q.BLOCK_1X16, device=dev, layout=IL)
    assert tuple(out.codes.shape) == (8, 32)
    short = q.NVFP4Tensor(out.codes[:6], out.scales, out.amax, out.s_enc, 6, 64, q.BLOCK_1X16,
                          layout=IL)  # the padding rows of the last group are missing
    with pytest.raises(ValueError):
        q.nvfp4_quantize(x, out=short)
    with pytest.raises(ValueError):
        q.alloc_nvfp4(32, 64, q.BLOCK_MX32, device=dev, layout=IL)
