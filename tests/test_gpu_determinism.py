"""Determinism across launch geometries: the same values reach the same bits
whatever grid the launch takes.

Recipe: "Pretraining Large Language Models with NVFP4" (gist.science
summary), Technische Zusammenfassung 2.A (tensor amax, block scales, codes)
and 2.B.2 (the GEMM passes).  A tensor maximum does not depend on the order
it is reduced in; a code depends only on its element, its block and the
tensor scale; each GEMM output element is one workgroup's fixed-order sum
over K.  So:
- amax by the flat pass (contiguous input) and by the row pass (padded
  leading dimension), and the RHT maximum by the fused pass and by the
  RHT quantiser's own pass, agree bit for bit;
- a tensor quantised whole and in row slices (different grids, the whole
  tensor's amax given) gives the same codes and scales (RNE);
- SR codes of a padded copy (another kernel path for the amax and another
  address pattern) equal those of the contiguous tensor;
- GEMM output rows computed in a launch over a row slice of A that is not
  tile-aligned (each element at another tile position) equal those rows of
  the launch over all of A, and likewise for a column slice of B.
"""
import numpy as np
import pytest

from tests.gpu_util import ensure_built, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    ensure_built()
    import quantize_precision_gemm_amd as q
    from quantize_precision_gemm_amd import workloads as wl
    dev = torch.device("cuda:0")
    return torch, q, wl, dev


def _padded(torch, x, pad=24):
    buf = torch.zeros((x.shape[0], x.shape[1] + pad), dtype=x.dtype, device=x.device)
    buf[:, : x.shape[1]] = x
    return buf[:, : x.shape[1]]


def _bits(t):
    import torch
    return t.view(torch.int32).item()


def test_amax_flat_rows_and_rht_paths_agree(env):
    torch, q, wl, dev = env
    x = to_dev(wl.lognormal_rows(np.random.default_rng(1), (1040, 4112)), dev)
    xp = _padded(torch, x)
    print("amax paths", flush=True)
    a_flat, _ = q.nvfp4_amax(x)
    a_rows, _ = q.nvfp4_amax(xp)
    mask = q.nvfp4_rht_sign_mask(5)
    a_d, ar_d = q.nvfp4_amax(x, mask)
    g = q.nvfp4_rht_quantize(x, mask, q.SR, 3)  # its own RHT amax pass
    torch.cuda.synchronize()
    assert _bits(a_flat) == _bits(a_rows) == _bits(a_d)
    assert _bits(ar_d) == _bits(g.amax)


@pytest.mark.parametrize("block", [0, 1])
def test_quantise_whole_vs_row_slices(env, block):
    torch, q, wl, dev = env
    x = to_dev(wl.student_t_unit_var(np.random.default_rng(2 + block), (1024, 2080), 4), dev)
    print(f"slices block={block}", flush=True)
    whole = q.nvfp4_quantize(x, block, q.RNE)
    amax = whole.amax
    srow = 16 if block == q.BLOCK_16X16 else 1
    for r0, r1 in [(0, 48), (48, 560), (560, 1024)]:
        part = q.nvfp4_quantize(x[r0:r1], block, q.RNE, amax_in=amax)
        torch.cuda.synchronize()
        assert torch.equal(part.codes[:, : 1040], whole.codes[r0:r1, : 1040])
        assert torch.equal(part.scales[:, : 2080 // 16], whole.scales[r0 // srow:r1 // srow, : 2080 // 16])


def test_sr_codes_padded_vs_contiguous(env):
    torch, q, wl, dev = env
    x = to_dev(wl.lognormal_rows(np.random.default_rng(4), (768, 3088)), dev)
    print("sr padded", flush=True)
    a = q.nvfp4_quantize(x, q.BLOCK_1X16, q.SR, 99)
    b = q.nvfp4_quantize(_padded(torch, x), q.BLOCK_1X16, q.SR, 99)
    mask = q.nvfp4_rht_sign_mask(7)
    c = q.nvfp4_rht_quantize(x, mask, q.SR, 98)
    d = q.nvfp4_rht_quantize(_padded(torch, x, 40), mask, q.SR, 98)
    torch.cuda.synchronize()
    for u, v in ((a, b), (c, d)):  # the logical columns (the buffers' row padding is not written)
        assert np.array_equal(u.codes_host(), v.codes_host())
        assert np.array_equal(u.scales_host(), v.scales_host())


def _slice_rows(q, t, r0, r1):
    """Rows r0..r1 of a 1x16 NVFP4 tensor as a tensor of its own (views of the buffers)."""
    return q.NVFP4Tensor(t.codes[r0:r1], t.scales[r0:r1], t.amax, t.s_enc, r1 - r0, t.cols, t.block)


@pytest.mark.parametrize("out_dtype", ["float32", "bfloat16"])
def test_gemm_rows_and_columns_independent_of_tiling(env, out_dtype):
    torch, q, wl, dev = env
    dt = getattr(torch, out_dtype)
    rng = np.random.default_rng(9)
    M, K, N = 1100, 1552, 900
    a = q.nvfp4_quantize(to_dev(wl.student_t_unit_var(rng, (M, K), 4), dev))
    b = q.nvfp4_quantize(to_dev(wl.normal(rng, (N, K), 0.02), dev))   # 1x16: row slices allowed
    print(f"gemm tiling {out_dtype}", flush=True)
    full = q.nvfp4_gemm(q.FPROP, a, b, dt)
    r0, r1 = 100, 612        # not 256-aligned: every element at another tile position
    rows = q.nvfp4_gemm(q.FPROP, _slice_rows(q, a, r0, r1), b, dt)
    c0, c1 = 37 * 16, 37 * 16 + 300
    cols = q.nvfp4_gemm(q.FPROP, a, _slice_rows(q, b, c0, c1), dt)
    torch.cuda.synchronize()
    iv = torch.int32 if dt == torch.float32 else torch.int16
    assert torch.equal(rows.view(iv), full[r0:r1].contiguous().view(iv))
    assert torch.equal(cols.view(iv), full[:, c0:c1].contiguous().view(iv))
