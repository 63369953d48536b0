"""Parity of the 4-block MLP training step at full size, as bench.py --workload
mlp runs it.

Workload: tokens 16384 (batch 4 x sequence 4096), hidden 5120, FFN 20480;
per block an up- (5120 -> 20480) and a down-projection (20480 -> 5120);
blocks 1-3 in NVFP4, block 4 kept in BF16 ("Pretraining Large Language Models
with NVFP4", gist.science summary, Technische Zusammenfassung 2.B.1 and
2.B.2); activations Student-t(3), seed 1; each layer has its own inputs.

After one step, every layer is checked against the oracle:
- NVFP4 layers: every code and every scale of all five quantised operands
  (X 1x16 RNE, W 16x16 RNE with the transposed copy dgrad reads, dY 1x16 SR,
  RHT(dY)^T SR, RHT(X)^T RNE) compared in full, bit for bit, with the
  oracle's quantisation of the whole tensor;
- every GEMM (18 NVFP4, 6 bf16) on 256 whole output rows, four from each
  256-row tile of the output (relative Frobenius <= 1e-5 on the kernel's fp32
  output), and the bf16 outputs of the step equal to round-to-nearest-even
  of that fp32 output over the whole matrix.
"""
import numpy as np
import pytest

from tests.gpu_util import ensure_built, rel_fro

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module")
def mlp():
    import torch
    ensure_built()
    import oracle
    import quantize_precision_gemm_amd as q
    import bench

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("building the MLP step", flush=True)
    step = bench.build_mlp_step(q, torch, dev)
    print("running one step", flush=True)
    step.run()
    torch.cuda.synchronize()
    return torch, oracle, q, step


def _host(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _f32(t):
    return np.float32(t.item())


def _sample_rows(n, seed, total=256):
    """`total` distinct output rows spread over every 256-row tile of [0, n)
    (the same count from each tile, tile-relative positions drawn with
    `seed`), always including the first and the last row."""
    tiles = (n + 255) // 256
    per = max(1, -(-total // tiles))
    rng = np.random.default_rng(seed)
    rows = []
    for t in range(tiles):
        lo, hi = 256 * t, min(256 * t + 256, n)
        rows.extend(lo + rng.choice(hi - lo, min(per, hi - lo), replace=False))
    rows = np.unique(np.concatenate([rows, [0, n - 1]]))
    if len(rows) > total:  # keep the spread: `total` evenly spaced picks, both ends included
        rows = rows[np.round(np.linspace(0, len(rows) - 1, total)).astype(int)]
    return rows


def _same(g, o, what, transposed=False):
    """Every code and scale of the device tensor g (its transposed copy if
    `transposed`) equals the oracle's o; codes read back in row-major order
    whatever the tensor's code layout."""
    gc = g.codes_t_host() if transposed else g.codes_host()
    g_scales = g.scales_t if transposed else g.scales
    if not np.array_equal(gc, o.codes):
        bad = np.argwhere(gc != o.codes)
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at {tuple(bad[0])}")
    gs = g_scales[:, : o.scales.shape[1]].cpu().numpy()
    if not np.array_equal(gs, o.scales):
        bad = np.argwhere(gs != o.scales)
        raise AssertionError(f"{what}: {len(bad)} scales differ, first at {tuple(bad[0])}")


def _check_scalars(g, o, what):
    assert _f32(g.amax) == np.float32(o.amax), f"{what}: amax {_f32(g.amax)} vs {o.amax}"
    assert _f32(g.s_enc) == np.float32(o.s_enc), f"{what}: s_enc {_f32(g.s_enc)} vs {o.s_enc}"


def _rows_err(torch, out32, rows, want):
    got = out32[torch.as_tensor(rows, device=out32.device)].double().cpu().numpy()
    return rel_fro(got, want)


def _check_nvfp4_layer(torch, oracle, q, L, idx):
    from quantize_precision_gemm_amd.step import SR_SEED_DY, SR_SEED_DY_RHT, RHT_SEED
    M, K, N = L.M, L.K, L.N
    tag = f"layer {idx} ({M}x{K} -> {N})"
    print(f"{tag}: copying inputs", flush=True)
    X, W, DY = _host(L.x), _host(L.w), _host(L.dy)
    assert L.mask == oracle.rht_sign_mask(L.seed + RHT_SEED)

    print(f"{tag}: X, W and W^T in full", flush=True)
    qx = oracle.quantize(X, oracle.BLOCK_1X16, oracle.RNE)
    _check_scalars(L.gx, qx, f"{tag} X")
    _same(L.gx, qx, f"{tag} X")
    qw = oracle.quantize(W, oracle.BLOCK_16X16, oracle.RNE)
    _check_scalars(L.gw, qw, f"{tag} W")
    _same(L.gw, qw, f"{tag} W")
    qwt = oracle.quantize(np.ascontiguousarray(W.T), oracle.BLOCK_16X16, oracle.RNE)
    _same(L.gw, qwt, f"{tag} W^T (dgrad operand)", transposed=True)
    del qwt
    print(f"{tag}: dY (SR) in full", flush=True)
    qdy = oracle.quantize(DY, oracle.BLOCK_1X16, oracle.SR, L.seed + SR_SEED_DY)
    _check_scalars(L.gdy, qdy, f"{tag} dY")
    _same(L.gdy, qdy, f"{tag} dY")
    print(f"{tag}: RHT operands in full", flush=True)
    qdyt = oracle.rht_quantize(DY, L.mask, oracle.SR, L.seed + SR_SEED_DY_RHT)
    _check_scalars(L.gdyt, qdyt, f"{tag} RHT(dY)^T")
    _same(L.gdyt, qdyt, f"{tag} RHT(dY)^T")
    qxt = oracle.rht_quantize(X, L.mask, oracle.RNE)
    _check_scalars(L.gxt, qxt, f"{tag} RHT(X)^T")
    _same(L.gxt, qxt, f"{tag} RHT(X)^T")
    del X, W, DY

    print(f"{tag}: GEMMs on 256 rows each", flush=True)
    y32 = q.nvfp4_gemm(q.FPROP, L.gx, L.gw, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), L.y), f"{tag}: fprop bf16 output"
    rows = _sample_rows(M, 10 * idx + 1)
    err = _rows_err(torch, y32, rows, oracle.gemm(oracle.FPROP, qx, qw, rows=rows))
    assert err <= TOL, f"{tag} fprop: relative Frobenius error {err:.3e} on {len(rows)} rows"
    del y32
    dx32 = q.nvfp4_gemm(q.DGRAD, L.gdy, L.gw, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(dx32.to(torch.bfloat16), L.dx), f"{tag}: dgrad bf16 output"
    rows = _sample_rows(M, 10 * idx + 2)
    err = _rows_err(torch, dx32, rows, oracle.gemm(oracle.DGRAD, qdy, qw, rows=rows))
    assert err <= TOL, f"{tag} dgrad: relative Frobenius error {err:.3e} on {len(rows)} rows"
    del dx32
    rows = _sample_rows(N, 10 * idx + 3)
    err = _rows_err(torch, L.dw, rows, oracle.gemm(oracle.WGRAD, qdyt, qxt, rows=rows))
    assert err <= TOL, f"{tag} wgrad: relative Frobenius error {err:.3e} on {len(rows)} rows"


def _check_bf16_layer(torch, oracle, q, L, idx):
    M, K, N = L.M, L.K, L.N
    tag = f"bf16 layer {idx} ({M}x{K} -> {N})"
    print(f"{tag}: GEMMs on 256 rows each", flush=True)
    W = _host(L.w)
    y32 = q.nvfp4_bf16_gemm(q.FPROP, L.x, L.w, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), L.y), f"{tag}: fprop bf16 output"
    rows = _sample_rows(M, 10 * idx + 1)
    rt = torch.as_tensor(rows, device=L.x.device)
    err = _rows_err(torch, y32, rows, oracle.bf16_gemm(oracle.FPROP, _host(L.x[rt]), W))
    assert err <= TOL, f"{tag} fprop: relative Frobenius error {err:.3e}"
    del y32
    dx32 = q.nvfp4_bf16_gemm(q.DGRAD, L.dy, L.w, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(dx32.to(torch.bfloat16), L.dx), f"{tag}: dgrad bf16 output"
    rows = _sample_rows(M, 10 * idx + 2)
    rt = torch.as_tensor(rows, device=L.x.device)
    err = _rows_err(torch, dx32, rows, oracle.bf16_gemm(oracle.DGRAD, _host(L.dy[rt]), W))
    assert err <= TOL, f"{tag} dgrad: relative Frobenius error {err:.3e}"
    del dx32, W
    rows = _sample_rows(N, 10 * idx + 3)
    rt = torch.as_tensor(rows, device=L.x.device)
    # rows n of dW = dY^T X are columns n of dY
    err = _rows_err(torch, L.dw, rows,
                    oracle.bf16_gemm(oracle.WGRAD, _host(L.dy[:, rt]), _host(L.x)))
    assert err <= TOL, f"{tag} wgrad: relative Frobenius error {err:.3e}"


def test_sample_rows_cover_every_tile():
    for n in (5120, 16384, 20480):
        rows = _sample_rows(n, 0)
        assert len(rows) == 256 and len(np.unique(rows)) == 256 and rows[0] == 0 and rows[-1] == n - 1
        assert len(set(rows // 256)) == (n + 255) // 256


def test_mlp_step_structure(mlp):
    torch, oracle, q, step = mlp
    from quantize_precision_gemm_amd.step import BF16Linear, NVFP4Linear
    from quantize_precision_gemm_amd import workloads as wl
    shapes = wl.mlp_layers()
    assert len(step.layers) == 8
    for i, (L, sh) in enumerate(zip(step.layers, shapes)):
        assert (L.M, L.K, L.N) == (16384, sh.K, sh.N)
        assert isinstance(L, BF16Linear if i >= 6 else NVFP4Linear)
    assert abs(step.flops() - 24 * 2.0 * 16384 * 5120 * 20480) < 1


@pytest.mark.parametrize("idx", range(8))
def test_mlp_layer(mlp, idx):
    torch, oracle, q, step = mlp
    L = step.layers[idx]
    if idx >= 6:
        _check_bf16_layer(torch, oracle, q, L, idx)
    else:
        _check_nvfp4_layer(torch, oracle, q, L, idx)
