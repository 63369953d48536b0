"""Parity of the 4-block MLP training step at full size, as bench.py --workload
mlp runs it.

Workload: tokens 16384 (batch 4 x sequence 4096), hidden 5120, FFN 20480;
per block an up- (5120 -> 20480) and a down-projection (20480 -> 5120);
blocks 1-3 in NVFP4, block 4 kept in BF16 ("Pretraining Large Language Models
with NVFP4", gist.science summary, Technische Zusammenfassung 2.B.1 and
2.B.2); activations Student-t(3), seed 1; each layer has its own inputs.

After one step, every layer is checked against the oracle on samples small
enough for the CPU: tensor maxima and encode scales of every quantised
operand over the whole tensors; codes and scales of sampled rows (of whole
16x16 tiles for W, of sampled channels for the RHT operands), quantised by
the oracle from those rows with the whole tensor's amax and, for stochastic
rounding, the rows' element-index offset; each GEMM on sampled blocks of its
output (relative Frobenius <= 1e-5 on the kernel's fp32 output, and the bf16
outputs of the step equal to round-to-nearest-even of it).
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


def _ranges(n, lens=(4, 3, 3)):
    """Three contiguous ranges: the start, the middle, the end of [0, n)."""
    a, b, c = lens
    mid = n // 2 + 5
    return [(0, a), (mid, mid + b), (n - c, n)]


def _check_quant_rows(g_codes, g_scales, o, r0, r1, what, scale_rows=None):
    gc = g_codes[r0:r1, : o.codes.shape[1]].cpu().numpy()
    np.testing.assert_array_equal(gc, o.codes, err_msg=f"{what}: codes rows {r0}:{r1}")
    s0, s1 = scale_rows if scale_rows else (r0, r1)
    gs = g_scales[s0:s1, : o.scales.shape[1]].cpu().numpy()
    np.testing.assert_array_equal(gs, o.scales, err_msg=f"{what}: scales rows {s0}:{s1}")


def _check_scalars(g, amax, oracle, what):
    assert _f32(g.amax) == np.float32(amax), f"{what}: amax {_f32(g.amax)} vs {amax}"
    s = oracle.tensor_scale(np.float32(amax))
    assert _f32(g.s_enc) == np.float32(s), f"{what}: s_enc {_f32(g.s_enc)} vs {s}"


def _blocks_err(pairs):
    got = np.concatenate([g.reshape(-1) for g, _ in pairs])
    want = np.concatenate([w.reshape(-1) for _, w in pairs])
    return rel_fro(got, want)


def _check_nvfp4_layer(torch, oracle, q, L, idx):
    from quantize_precision_gemm_amd.step import SR_SEED_DY, SR_SEED_DY_RHT, RHT_SEED
    M, K, N = L.M, L.K, L.N
    tag = f"layer {idx} ({M}x{K} -> {N})"
    print(f"{tag}: copying inputs", flush=True)
    X, W, DY = _host(L.x), _host(L.w), _host(L.dy)
    assert L.mask == oracle.rht_sign_mask(L.seed + RHT_SEED)

    print(f"{tag}: tensor maxima", flush=True)
    aX, aW, aDY = oracle.amax(X), oracle.amax(W), oracle.amax(DY)
    aXr, aDYr = oracle.rht_amax(X, L.mask), oracle.rht_amax(DY, L.mask)
    _check_scalars(L.gx, aX, oracle, f"{tag} X")
    _check_scalars(L.gw, aW, oracle, f"{tag} W")
    _check_scalars(L.gdy, aDY, oracle, f"{tag} dY")
    _check_scalars(L.gxt, aXr, oracle, f"{tag} RHT(X)")
    _check_scalars(L.gdyt, aDYr, oracle, f"{tag} RHT(dY)")

    print(f"{tag}: sampled quantisations", flush=True)
    m_rng = _ranges(M)
    qx = {r: oracle.quantize(X[r[0]:r[1]], amax_in=aX) for r in m_rng}
    qdy = {r: oracle.quantize(DY[r[0]:r[1]], oracle.BLOCK_1X16, oracle.SR, L.seed + SR_SEED_DY,
                              amax_in=aDY, idx0=r[0] * N) for r in m_rng}
    for r in m_rng:
        _check_quant_rows(L.gx.codes, L.gx.scales, qx[r], r[0], r[1], f"{tag} X")
        _check_quant_rows(L.gdy.codes, L.gdy.scales, qdy[r], r[0], r[1], f"{tag} dY")
    n_grp = [(0, 16), (N - 16, N)]       # whole 16x16 tiles of W by rows (fprop)
    k_grp = [(0, 16), (K - 16, K)]       # and by columns (dgrad)
    qw_rows = {g: oracle.quantize(W[g[0]:g[1]], oracle.BLOCK_16X16, amax_in=aW) for g in n_grp}
    for g in n_grp:
        _check_quant_rows(L.gw.codes, L.gw.scales, qw_rows[g], g[0], g[1], f"{tag} W",
                          (g[0] // 16, g[1] // 16))
    qw_cols = {g: oracle.quantize(np.ascontiguousarray(W[:, g[0]:g[1]]), oracle.BLOCK_16X16,
                                  amax_in=aW) for g in k_grp}
    for g in k_grp:   # the transposed copy dgrad reads: tiles of W^T
        ot = oracle.quantize(np.ascontiguousarray(W[:, g[0]:g[1]].T), oracle.BLOCK_16X16,
                             amax_in=aW)
        _check_quant_rows(L.gw.codes_t, L.gw.scales_t, ot, g[0], g[1], f"{tag} W^T",
                          (g[0] // 16, g[1] // 16))
    n_rng = _ranges(N, (3, 2, 2))
    k_rng = _ranges(K, (2, 3, 2))
    qdyt = {r: oracle.rht_quantize(np.ascontiguousarray(DY[:, r[0]:r[1]]), L.mask, oracle.SR,
                                   L.seed + SR_SEED_DY_RHT, amax_in=aDYr, idx0=r[0] * M)
            for r in n_rng}
    qxt = {r: oracle.rht_quantize(np.ascontiguousarray(X[:, r[0]:r[1]]), L.mask, oracle.RNE,
                                  amax_in=aXr) for r in k_rng}
    for r in n_rng:
        _check_quant_rows(L.gdyt.codes, L.gdyt.scales, qdyt[r], r[0], r[1], f"{tag} RHT(dY)^T")
    for r in k_rng:
        _check_quant_rows(L.gxt.codes, L.gxt.scales, qxt[r], r[0], r[1], f"{tag} RHT(X)^T")
    del X, W, DY

    print(f"{tag}: sampled GEMM blocks", flush=True)
    y32 = q.nvfp4_gemm(q.FPROP, L.gx, L.gw, torch.float32)
    dx32 = q.nvfp4_gemm(q.DGRAD, L.gdy, L.gw, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), L.y), f"{tag}: fprop bf16 output"
    assert torch.equal(dx32.to(torch.bfloat16), L.dx), f"{tag}: dgrad bf16 output"
    fp = [(y32[r[0]:r[1], g[0]:g[1]].double().cpu().numpy(),
           oracle.gemm(oracle.FPROP, qx[r], qw_rows[g])) for r in m_rng for g in n_grp]
    dg = [(dx32[r[0]:r[1], g[0]:g[1]].double().cpu().numpy(),
           oracle.gemm(oracle.DGRAD, qdy[r], qw_cols[g])) for r in m_rng for g in k_grp]
    wg = [(L.dw[a[0]:a[1], b[0]:b[1]].double().cpu().numpy(),
           oracle.gemm(oracle.WGRAD, qdyt[a], qxt[b])) for a in n_rng for b in k_rng]
    del y32, dx32
    for name, pairs in (("fprop", fp), ("dgrad", dg), ("wgrad", wg)):
        err = _blocks_err(pairs)
        assert err <= TOL, f"{tag} {name}: relative Frobenius error {err:.3e}"


def _check_bf16_layer(torch, oracle, q, L, idx):
    M, K, N = L.M, L.K, L.N
    tag = f"bf16 layer {idx} ({M}x{K} -> {N})"
    print(f"{tag}: sampled GEMM blocks", flush=True)
    m_rng, n_rng, k_rng = _ranges(M), _ranges(N, (3, 2, 2)), _ranges(K, (2, 3, 2))
    y32 = q.nvfp4_bf16_gemm(q.FPROP, L.x, L.w, torch.float32)
    dx32 = q.nvfp4_bf16_gemm(q.DGRAD, L.dy, L.w, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), L.y), f"{tag}: fprop bf16 output"
    assert torch.equal(dx32.to(torch.bfloat16), L.dx), f"{tag}: dgrad bf16 output"
    X = {r: _host(L.x[r[0]:r[1]]) for r in m_rng}
    DY = {r: _host(L.dy[r[0]:r[1]]) for r in m_rng}
    Wn = {r: _host(L.w[r[0]:r[1]]) for r in n_rng}
    Wk = {r: _host(L.w[:, r[0]:r[1]]) for r in k_rng}
    DYn = {r: _host(L.dy[:, r[0]:r[1]]) for r in n_rng}
    Xk = {r: _host(L.x[:, r[0]:r[1]]) for r in k_rng}
    fp = [(y32[a[0]:a[1], b[0]:b[1]].double().cpu().numpy(),
           oracle.bf16_gemm(oracle.FPROP, X[a], Wn[b])) for a in m_rng for b in n_rng]
    dg = [(dx32[a[0]:a[1], b[0]:b[1]].double().cpu().numpy(),
           oracle.bf16_gemm(oracle.DGRAD, DY[a], Wk[b])) for a in m_rng for b in k_rng]
    wg = [(L.dw[a[0]:a[1], b[0]:b[1]].double().cpu().numpy(),
           oracle.bf16_gemm(oracle.WGRAD, DYn[a], Xk[b])) for a in n_rng for b in k_rng]
    del y32, dx32
    for name, pairs in (("fprop", fp), ("dgrad", dg), ("wgrad", wg)):
        err = _blocks_err(pairs)
        assert err <= TOL, f"{tag} {name}: relative Frobenius error {err:.3e}"


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
