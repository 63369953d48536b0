"""Parity of the MXFP4 comparison path (nvfp4_mx_quantize, nvfp4_mx_gemm)
with the oracle: codes and scales bit for bit in all three layouts, the GEMM
within 1e-5 relative Frobenius on fp32 output (bf16 output = RNE of the same
kernel's fp32 result), at sizes spanning several tiles with ragged tails and
at the 12B-layer shapes (sampled output rows)."""
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
    return torch, oracle, q, wl, torch.device("cuda:0")


def _same(g, o, what):
    gc, gs = g.codes_host(), g.scales_host()
    assert (g.rows, g.cols, g.block) == (o.rows, o.cols, 2), what
    if not np.array_equal(gc, o.codes):
        bad = np.argwhere(gc != o.codes)
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first ({r},{c}): "
                             f"gpu {gc[r, c]:#04x} oracle {o.codes[r, c]:#04x}")
    if not np.array_equal(gs, o.scales):
        bad = np.argwhere(gs != o.scales)
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} scales differ, first ({r},{c}): "
                             f"gpu {gs[r, c]} oracle {o.scales[r, c]}")


def _bits(wl, rng, shape, kind):
    if kind == "normal":
        return wl.normal(rng, shape, 1.0)
    if kind == "rows":
        return wl.lognormal_rows(rng, shape)
    x = rng.standard_normal(shape) * np.exp(rng.uniform(-40, 40, shape))
    return wl.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("shape", [(1, 32), (37, 96), (300, 1056), (256, 4096)])
@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("kind", ["normal", "rows", "wide"])
def test_mx_quantize_rows(env, shape, rounding, kind):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(shape[0] * 13 + shape[1] + rounding)
    x = _bits(wl, rng, shape, kind)
    print(f"mx rows {shape} r={rounding} {kind}", flush=True)
    g = q.nvfp4_mx_quantize(to_dev(x, dev), q.MX_ROWS, 0, rounding, 77)
    torch.cuda.synchronize()
    _same(g, oracle.mx_quantize(x, oracle.MX_ROWS, 0, rounding, 77), f"rows {shape}")


@pytest.mark.parametrize("shape", [(32, 8), (64, 24), (288, 200), (512, 264), (4096, 64)])
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("rounding", [0, 1])
def test_mx_quantize_cols(env, shape, mode, rounding):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(shape[0] + 5 * shape[1] + 3 * mode + rounding)
    x = _bits(wl, rng, shape, "rows" if rounding else "normal")
    mask = int(rng.integers(0, 65536))
    print(f"mx cols {shape} mode={mode} r={rounding}", flush=True)
    g = q.nvfp4_mx_quantize(to_dev(x, dev), mode, mask, rounding, 5)
    torch.cuda.synchronize()
    _same(g, oracle.mx_quantize(x, mode, mask, rounding, 5), f"cols {shape} mode {mode}")


def test_mx_quantize_strided_and_edges(env):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(3)
    full = wl.normal(rng, (96, 160), 1.0)
    x = np.ascontiguousarray(full[:, :128])
    xd = to_dev(full, dev)[:, :128]
    print("mx strided", flush=True)
    for mode in (0, 1, 2):
        g = q.nvfp4_mx_quantize(xd, mode, 0x2468, 1, 9)
        torch.cuda.synchronize()
        _same(g, oracle.mx_quantize(x, mode, 0x2468, 1, 9), f"strided mode {mode}")
    z = np.zeros((64, 64), np.uint16)
    z[3, 5] = 0x8000          # -0
    z[7, 40] = 0x0001         # smallest subnormal
    z[33, 2] = 0x0050
    big = np.zeros((64, 64), np.float32)
    big[0, 0] = 3.0e38
    big[40, 33] = -7.5
    big[41, 33] = 1e-30
    for name, xe in [("zero_subnormal", z), ("huge", wl.f32_to_bf16_bits(big))]:
        for mode in (0, 1, 2):
            for rounding in (0, 1):
                print(f"mx edge {name} mode={mode} r={rounding}", flush=True)
                g = q.nvfp4_mx_quantize(to_dev(xe, dev), mode, 0xBEEF, rounding, 3)
                torch.cuda.synchronize()
                _same(g, oracle.mx_quantize(xe, mode, 0xBEEF, rounding, 3), f"{name} {mode}")


def test_mx_empty_and_errors(env):
    torch, oracle, q, wl, dev = env
    print("mx empty / errors", flush=True)
    g = q.nvfp4_mx_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device=dev))
    assert (g.rows, g.cols) == (0, 64)
    g = q.nvfp4_mx_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device=dev), q.MX_COLS)
    assert (g.rows, g.cols) == (64, 0)
    x = torch.zeros((64, 48), dtype=torch.bfloat16, device=dev)
    with pytest.raises(RuntimeError, match="status -2"):
        q.nvfp4_mx_quantize(x)                      # 48 columns: not whole blocks of 32
    with pytest.raises(RuntimeError, match="status -2"):
        q.nvfp4_mx_quantize(x[:48], q.MX_COLS)      # 48 rows: not whole blocks of 32
    with pytest.raises(RuntimeError, match="status -4"):
        q.nvfp4_mx_quantize(x[:, :32], 3)
    a = q.nvfp4_mx_quantize(x[:, :32])
    b = q.nvfp4_mx_quantize(torch.zeros((16, 64), dtype=torch.bfloat16, device=dev))
    with pytest.raises(RuntimeError, match="status -5"):
        q.nvfp4_mx_gemm(a, b)                       # K 32 vs 64
    n = q.nvfp4_quantize(x[:, :32])
    with pytest.raises(RuntimeError, match="status -5"):
        q.nvfp4_mx_gemm(a, n)                       # an NVFP4 operand
    with pytest.raises(RuntimeError, match="status -4"):
        q.nvfp4_gemm(q.FPROP, n, a)                 # and the reverse
    c = q.nvfp4_mx_gemm(a, q.nvfp4_mx_quantize(torch.zeros((0, 32), dtype=torch.bfloat16, device=dev)))
    assert c.shape == (64, 0)
    torch.cuda.synchronize()


def _check_gemm(env, qa, qb, oa, ob, rows, what):
    torch, oracle, q, wl, dev = env
    c32 = q.nvfp4_mx_gemm(qa, qb, torch.float32)
    c16 = q.nvfp4_mx_gemm(qa, qb, torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.mx_gemm(oa, ob, rows)
    got = c32.cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[rows]
    err = rel_fro(got, ref)
    assert err <= TOL, f"{what}: rel Frobenius {err:.3e}"
    bits = c16.cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, bf16_rne_bits(c32.cpu().numpy()), err_msg=f"{what} bf16")
    return err


@pytest.mark.parametrize("MNK", [(32, 32, 32), (256, 256, 256), (300, 200, 96), (520, 264, 1056),
                                 (64, 48, 4128), (1, 8, 160)])
@pytest.mark.parametrize("rounding", [0, 1])
def test_mx_gemm(env, MNK, rounding):
    torch, oracle, q, wl, dev = env
    M, N, K = MNK
    rng = np.random.default_rng(M + N + K + rounding)
    a = wl.lognormal_rows(rng, (M, K)) if rounding else wl.normal(rng, (M, K), 1.0)
    b = wl.normal(rng, (N, K), 0.05)
    print(f"mx gemm {MNK} r={rounding}", flush=True)
    qa = q.nvfp4_mx_quantize(to_dev(a, dev), q.MX_ROWS, 0, rounding, 4)
    qb = q.nvfp4_mx_quantize(to_dev(b, dev))
    oa = oracle.mx_quantize(a, oracle.MX_ROWS, 0, rounding, 4)
    ob = oracle.mx_quantize(b)
    _same(qa, oa, "a")
    _same(qb, ob, "b")
    _check_gemm(env, qa, qb, oa, ob, None, f"gemm {MNK}")


# Contraction lengths around the kernel's switch to loading three steps'
# scales at once (taken while 9 or more whole 128-element steps remain):
# 8 to 16 whole steps, with and without a partial last step.
@pytest.mark.parametrize("K", [1024, 1056, 1152, 1184, 1280, 1536, 1920, 2048, 2080])
def test_mx_gemm_scale_load_switch(env, K):
    torch, oracle, q, wl, dev = env
    M, N = 264, 520
    rng = np.random.default_rng(K)
    a = wl.lognormal_rows(rng, (M, K))
    b = wl.normal(rng, (N, K), 0.05)
    print(f"mx gemm scale-load switch K={K}", flush=True)
    qa = q.nvfp4_mx_quantize(to_dev(a, dev), q.MX_ROWS, 0, 1, 4)
    qb = q.nvfp4_mx_quantize(to_dev(b, dev))
    oa = oracle.mx_quantize(a, oracle.MX_ROWS, 0, 1, 4)
    ob = oracle.mx_quantize(b)
    _same(qa, oa, "a")
    _same(qb, ob, "b")
    _check_gemm(env, qa, qb, oa, ob, None, f"gemm K={K}")


def test_mx_gemm_padded_leading_dimensions(env):
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(12)
    M, N, K = 72, 40, 224
    a, b = wl.normal(rng, (M, K), 1.0), wl.normal(rng, (N, K), 1.0)
    print("mx gemm padded", flush=True)
    qa = q.alloc_nvfp4(M, K + 96, q.BLOCK_MX32, device=dev)   # wider rows than needed
    qb = q.alloc_nvfp4(N, K + 32, q.BLOCK_MX32, device=dev)
    qa.codes.fill_(0x77)                                       # garbage past K must not count
    qb.codes.fill_(0x77)
    q.nvfp4_mx_quantize(to_dev(a, dev), out=qa)
    q.nvfp4_mx_quantize(to_dev(b, dev), out=qb)
    out = torch.empty((M, N + 12), dtype=torch.float32, device=dev)
    c = q.nvfp4_mx_gemm(qa, qb, out=out[:, :N])
    torch.cuda.synchronize()
    ref = oracle.mx_gemm(oracle.mx_quantize(a), oracle.mx_quantize(b))
    assert rel_fro(c.cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("pass_", ["fprop", "dgrad", "wgrad"])
def test_mx_gemm_full_size(env, pass_):
    # the 12B-layer passes in MXFP4: X 8192x5120, W 20480x5120, dY 8192x20480;
    # operands quantised in the layout each pass contracts over; 40 sampled
    # output rows against the oracle
    torch, oracle, q, wl, dev = env
    M, K, N = 8192, 5120, 20480
    rng = np.random.default_rng({"fprop": 1, "dgrad": 2, "wgrad": 3}[pass_])
    mask = oracle.rht_sign_mask(1000)
    print(f"mx full {pass_}: inputs", flush=True)
    if pass_ == "fprop":
        a, b = wl.student_t_unit_var(rng, (M, K), 3), wl.normal(rng, (N, K), 0.02)
        ma, mb, ra, rb = 0, 0, 0, 0
    elif pass_ == "dgrad":
        a, b = wl.normal(rng, (M, N), 1e-3), wl.normal(rng, (N, K), 0.02)
        ma, mb, ra, rb = 0, 1, 1, 0
    else:
        a, b = wl.normal(rng, (M, N), 1e-3), wl.student_t_unit_var(rng, (M, K), 3)
        ma, mb, ra, rb = 2, 2, 1, 0
    qa = q.nvfp4_mx_quantize(to_dev(a, dev), ma, mask, ra, 100)
    qb = q.nvfp4_mx_quantize(to_dev(b, dev), mb, mask, rb, 101)
    torch.cuda.synchronize()
    print(f"mx full {pass_}: oracle", flush=True)
    oa = oracle.mx_quantize(a, ma, mask, ra, 100)
    ob = oracle.mx_quantize(b, mb, mask, rb, 101)
    _same(qa, oa, f"{pass_} a")
    _same(qb, ob, f"{pass_} b")
    rows = np.unique(np.concatenate([[0, qa.rows - 1], rng.choice(qa.rows, 40, replace=False)]))
    print(f"mx full {pass_}: gemm", flush=True)
    _check_gemm(env, qa, qb, oa, ob, rows, f"{pass_} full")


def test_mx_training_step(env):
    # the MXFP4 layer of the training step runs exactly the calls it names:
    # its outputs equal the library calls made one by one (bit for bit) and
    # the oracle's MXFP4 passes (within the GEMM tolerance)
    torch, oracle, q, wl, dev = env
    from quantize_precision_gemm_amd.step import MXFP4Linear, TrainingStep, SR_SEED_DY, SR_SEED_DY_RHT
    rng = np.random.default_rng(33)
    M, K, N, seed = 512, 384, 640, 7
    xb, wb, dyb = wl.normal(rng, (M, K), 1.0), wl.normal(rng, (N, K), 0.02), wl.lognormal_rows(rng, (M, N))
    x, w, dy = to_dev(xb, dev), to_dev(wb, dev), to_dev(dyb, dev)
    print("mx training step", flush=True)
    layer = MXFP4Linear(q, torch, x, w, dy, seed)
    TrainingStep(torch, [layer], dev).run()
    mask = layer.mask
    y = q.nvfp4_mx_gemm(q.nvfp4_mx_quantize(x), q.nvfp4_mx_quantize(w))
    dx = q.nvfp4_mx_gemm(q.nvfp4_mx_quantize(dy, q.MX_ROWS, 0, q.SR, seed + SR_SEED_DY),
                         q.nvfp4_mx_quantize(w, q.MX_COLS))
    dw = q.nvfp4_mx_gemm(q.nvfp4_mx_quantize(dy, q.MX_COLS_RHT, mask, q.SR, seed + SR_SEED_DY_RHT),
                         q.nvfp4_mx_quantize(x, q.MX_COLS_RHT, mask), torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(layer.y, y) and torch.equal(layer.dx, dx) and torch.equal(layer.dw, dw)
    odw = oracle.mx_gemm(oracle.mx_quantize(dyb, oracle.MX_COLS_RHT, mask, oracle.SR, seed + SR_SEED_DY_RHT),
                         oracle.mx_quantize(xb, oracle.MX_COLS_RHT, mask))
    assert rel_fro(layer.dw.cpu().numpy(), odw) <= TOL
