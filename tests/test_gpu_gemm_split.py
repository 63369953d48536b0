"""GPU parity of nvfp4_gemm_split: the NVFP4 GEMM whose last, partial wave
of output tiles is computed in parts along the contraction (fp32 partial
sums in a workspace, added in part order by a second kernel).

Passes: "Pretraining Large Language Models with NVFP4" (gist.science
summary), Technische Zusammenfassung 2.B.2 (Fprop, Dgrad, Wgrad).  The split
changes only the fp32 accumulation order, so the bar is the GEMM's: relative
Frobenius error <= 1e-5 against the fp64 oracle on the fp32 output, and the
bf16 output equal to round-to-nearest-even of the same call's fp32 output.
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


def _cus(torch, dev):
    return torch.cuda.get_device_properties(dev).multi_processor_count


def _check(torch, q, pass_, ga, gb, want, rows=None):
    """Both output dtypes of the split call: fp32 within TOL of the oracle
    (on `rows` if given), bf16 = RNE of that fp32, two calls identical."""
    ws = q.nvfp4_gemm_split_workspace(pass_, ga, gb)
    buf = torch.empty(max(ws, 1), dtype=torch.uint8, device=ga.codes.device)
    y32 = q.nvfp4_gemm_split(pass_, ga, gb, buf, torch.float32)
    y32b = q.nvfp4_gemm_split(pass_, ga, gb, buf, torch.float32)
    y16 = q.nvfp4_gemm_split(pass_, ga, gb, buf, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y32.view(torch.int32), y32b.view(torch.int32)), "not deterministic"
    if rows is None:
        g32 = y32.cpu().numpy()
        b16 = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        rt = torch.as_tensor(rows, device=y32.device)
        g32 = y32[rt].cpu().numpy()
        b16 = y16[rt].view(torch.int16).cpu().numpy().view(np.uint16)
    err = rel_fro(g32, want)
    assert err <= TOL, f"relative Frobenius error {err:.3e}"
    np.testing.assert_array_equal(b16, bf16_rne_bits(g32))
    return ws, y32


# (pass, M, K, N): small grids that leave a partial wave on any device with
# more compute units than tiles, ragged tiles, a K tail (K % 64 = 16)
SMALL = [("fprop", 300, 4112, 528), ("dgrad", 272, 2064, 4128), ("wgrad", 528, 3088, 96)]


@pytest.mark.parametrize("case", SMALL)
def test_split_small(env, case):
    torch, oracle, q, wl, dev = env
    name, M, K, N = case
    rng = np.random.default_rng(M + K + N)
    print(f"split {case}", flush=True)
    if name == "fprop":
        x, w = wl.student_t_unit_var(rng, (M, K), 4), wl.normal(rng, (N, K), 0.02)
        ga, gb = q.nvfp4_quantize(to_dev(x, dev)), q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16)
        want, P = oracle.gemm(oracle.FPROP, oracle.quantize(x), oracle.quantize(w, oracle.BLOCK_16X16)), q.FPROP
    elif name == "dgrad":  # dX (M x K) = dY (M x N) W (N x K)
        dy, w = wl.lognormal_rows(rng, (M, N)), wl.normal(rng, (N, K), 0.02)
        ga = q.nvfp4_quantize(to_dev(dy, dev), q.BLOCK_1X16, q.SR, 5)
        gb = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, with_transpose=True)
        want = oracle.gemm(oracle.DGRAD, oracle.quantize(dy, oracle.BLOCK_1X16, oracle.SR, 5),
                           oracle.quantize(w, oracle.BLOCK_16X16))
        P = q.DGRAD
    else:  # dW (N x K) over M tokens
        dy, x = wl.lognormal_rows(rng, (M, N)), wl.student_t_unit_var(rng, (M, K), 4)
        mask = q.nvfp4_rht_sign_mask(3)
        ga, gb = q.nvfp4_rht_quantize(to_dev(dy, dev), mask, q.SR, 7), q.nvfp4_rht_quantize(to_dev(x, dev), mask)
        want = oracle.gemm(oracle.WGRAD, oracle.rht_quantize(dy, mask, oracle.SR, 7), oracle.rht_quantize(x, mask))
        P = q.WGRAD
    ws, _ = _check(torch, q, P, ga, gb, want)
    tiles = ((want.shape[0] + 255) // 256) * ((want.shape[1] + 255) // 256)
    if tiles % _cus(torch, dev) != 0:
        assert ws > 0  # the split path ran


# K for 6 output tiles (300 x 528) whose step counts (13, 21, 26 with a K
# tail, 29) leave 3, 5, 6 and 7 parts of at least 4 steps on 256 CUs: with
# 2, 4 and 8 above, every part count the plan can choose
PARTS = [(832, 3), (1344, 5), (1616, 6), (1856, 7)]


@pytest.mark.parametrize("K,parts", PARTS)
def test_split_part_counts(env, K, parts):
    torch, oracle, q, wl, dev = env
    M, N = 300, 528
    print(f"split parts K={K}", flush=True)
    rng = np.random.default_rng(K)
    x, w = wl.student_t_unit_var(rng, (M, K), 4), wl.normal(rng, (N, K), 0.02)
    ga, gb = q.nvfp4_quantize(to_dev(x, dev)), q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16)
    want = oracle.gemm(oracle.FPROP, oracle.quantize(x), oracle.quantize(w, oracle.BLOCK_16X16))
    ws, _ = _check(torch, q, q.FPROP, ga, gb, want)
    if _cus(torch, dev) == 256:  # 6 leftover tiles, `parts` parts of 256 x 256 fp32 each
        assert ws == 6 * parts * 256 * 256 * 4


@pytest.fixture(scope="module")
def layer(env):
    torch, oracle, q, wl, dev = env
    import bench
    print("12B layer step", flush=True)
    data, step = bench.build_layer_step(q, torch, dev)
    step.run()
    torch.cuda.synchronize()
    return data, step.layers[0]


def _rows(n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, 48, replace=False)]))


def test_split_12b_dgrad_and_wgrad(env, layer):
    # 640 dgrad tiles and 1600 wgrad tiles: partial last waves on 256 CUs
    torch, oracle, q, wl, dev = env
    import bench
    data, L = layer
    mask = L.mask
    print("oracle operands", flush=True)
    ody = oracle.quantize(data["dY"], oracle.BLOCK_1X16, oracle.SR, bench.SEED + 100)
    ow = oracle.quantize(data["W"], oracle.BLOCK_16X16)
    rows = _rows(bench.M, 1)
    ws, _ = _check(torch, q, q.DGRAD, L.gdy, L.gw, oracle.gemm(oracle.DGRAD, ody, ow, rows=rows), rows)
    if _cus(torch, dev) == 256:
        assert ws == 128 * 2 * 256 * 256 * 4  # 128 leftover tiles in 2 parts
    del ody, ow
    odyt = oracle.rht_quantize(data["dY"], mask, oracle.SR, bench.SEED + 101)
    oxt = oracle.rht_quantize(data["X"], mask, oracle.RNE)
    rows = _rows(bench.N, 2)
    ws, _ = _check(torch, q, q.WGRAD, L.gdyt, L.gxt, oracle.gemm(oracle.WGRAD, odyt, oxt, rows=rows), rows)
    if _cus(torch, dev) == 256:
        assert ws == 64 * 4 * 256 * 256 * 4   # 64 leftover tiles in 4 parts


def test_no_partial_wave_is_nvfp4_gemm(env, layer):
    # fprop at the 12B shape fills whole waves (2560 tiles on 256 CUs): no
    # workspace, and the call is nvfp4_gemm (bit-identical output)
    torch, oracle, q, wl, dev = env
    data, L = layer
    if (2560 % _cus(torch, dev)) != 0:
        pytest.skip("tile count not a multiple of this device's compute units")
    assert q.nvfp4_gemm_split_workspace(q.FPROP, L.gx, L.gw) == 0
    a = q.nvfp4_gemm(q.FPROP, L.gx, L.gw, torch.bfloat16)
    b = q.nvfp4_gemm_split(q.FPROP, L.gx, L.gw, None, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_split_workspace_errors(env):
    torch, oracle, q, wl, dev = env
    import ctypes
    rng = np.random.default_rng(3)
    x, w = wl.normal(rng, (300, 4112), 1.0), wl.normal(rng, (528, 4112), 0.02)
    ga, gb = q.nvfp4_quantize(to_dev(x, dev)), q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16)
    need = q.nvfp4_gemm_split_workspace(q.FPROP, ga, gb)
    assert need > 0
    small = torch.empty(need - 16, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError):  # the binding checks the size first
        q.nvfp4_gemm_split(q.FPROP, ga, gb, small)
    c = torch.full((300, 528), 5.0, dtype=torch.float32, device=dev)
    da, db = ga.descriptor(), gb.descriptor()
    L = q.load_library()
    s = torch.cuda.current_stream().cuda_stream
    assert L.nvfp4_gemm_split(q.FPROP, ctypes.byref(da), ctypes.byref(db), c.data_ptr(), 528,
                              q.OUT_FP32, small.data_ptr(), need - 16, s) == -7
    assert L.nvfp4_gemm_split(q.FPROP, ctypes.byref(da), ctypes.byref(db), c.data_ptr(), 528,
                              q.OUT_FP32, None, 0, s) == -7
    torch.cuda.synchronize()
    assert (c == 5.0).all().item()  # nothing was launched


def test_binding_noalloc_equals_split(env):
    # the binding's nvfp4_gemm_split_noalloc runs the same kernels as
    # nvfp4_gemm_split with a caller workspace: identical output
    torch, oracle, q, wl, dev = env
    rng = np.random.default_rng(21)
    x, w = wl.normal(rng, (300, 4112), 1.0), wl.normal(rng, (528, 4112), 0.02)
    ga, gb = q.nvfp4_quantize(to_dev(x, dev)), q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16)
    print("binding noalloc", flush=True)
    a = q.nvfp4_gemm_split_noalloc(q.FPROP, ga, gb, torch.float32)
    b = q.nvfp4_gemm_split(q.FPROP, ga, gb, None, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
