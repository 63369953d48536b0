"""GPU parity of the bf16 GEMM (the layers that keep BF16) against the fp64 oracle.

Bar: relative Frobenius error <= 1e-5 on the kernel's fp32 output (bf16
products are exact in fp32; only the fp32 accumulation rounds); the bf16
output is bit-equal to round-to-nearest-even of that fp32 output.
Source: "Pretraining Large Language Models with NVFP4" (gist.science
summary), Technische Zusammenfassung 2.B.1 (a few linear layers stay in
BF16) with the three passes of 2.B.2.
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


def _operands(wl, pass_, M, K, N, seed):
    rng = np.random.default_rng(seed)
    x = wl.student_t_unit_var(rng, (M, K), 3)
    w = wl.normal(rng, (N, K), 0.02)
    dy = wl.lognormal_rows(rng, (M, N))
    return {0: (x, w), 1: (dy, w), 2: (dy, x)}[pass_]


def _run(torch, q, pass_, a, b, want, out_pad=0):
    dt = [torch.float32, torch.bfloat16]
    outs = []
    for d in dt:
        if out_pad:
            shape = want.shape
            buf = torch.full((shape[0], shape[1] + out_pad), -7.0, dtype=d, device=a.device)
            q.nvfp4_bf16_gemm(pass_, a, b, out=buf[:, : shape[1]])
            outs.append(buf)
        else:
            outs.append(q.nvfp4_bf16_gemm(pass_, a, b, d))
    torch.cuda.synchronize()
    n = want.shape[1]
    g32 = outs[0][:, :n].cpu().numpy()
    err = rel_fro(g32, want)
    assert err <= TOL, f"relative Frobenius error {err:.3e}"
    b16 = outs[1][:, :n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(b16, bf16_rne_bits(g32))
    if out_pad:  # nothing written past the logical columns
        assert (outs[0][:, n:] == -7.0).all().item() and (outs[1][:, n:] == -7.0).all().item()
    return g32


# (M, K, N), multiples of 8: one tile, ragged tiles on every side, K steps
# with a partial last step (K % 64 != 0), a long contraction
SHAPES = [(8, 8, 8), (24, 72, 40), (264, 200, 520), (512, 512, 768), (1032, 136, 264),
          (64, 4104, 96)]
PASSES = {"fprop": 0, "dgrad": 1, "wgrad": 2}


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("name", list(PASSES))
def test_bf16_gemm(env, name, shape):
    torch, oracle, q, wl, dev = env
    pass_ = PASSES[name]
    M, K, N = shape
    print(f"bf16 {name} {shape}", flush=True)
    a, b = _operands(wl, pass_, M, K, N, M + 3 * K + 7 * N + pass_)
    want = oracle.bf16_gemm(pass_, a, b)
    _run(torch, q, pass_, to_dev(a, dev), to_dev(b, dev), want)


@pytest.mark.parametrize("name", list(PASSES))
def test_bf16_gemm_strided(env, name):
    # operands are column slices of wider tensors; the output has a wider row
    torch, oracle, q, wl, dev = env
    pass_ = PASSES[name]
    M, K, N = 272, 152, 328
    a, b = _operands(wl, pass_, M, K, N, 99 + pass_)
    want = oracle.bf16_gemm(pass_, a, b)
    pad = 24
    A = torch.zeros((a.shape[0], a.shape[1] + pad), dtype=torch.bfloat16, device=dev)
    B = torch.zeros((b.shape[0], b.shape[1] + pad), dtype=torch.bfloat16, device=dev)
    A[:, : a.shape[1]] = to_dev(a, dev)
    B[:, : b.shape[1]] = to_dev(b, dev)
    _run(torch, q, pass_, A[:, : a.shape[1]], B[:, : b.shape[1]], want, out_pad=16)


def test_bf16_gemm_empty(env):
    torch, oracle, q, wl, dev = env
    # empty contraction: the output is all zero
    x = torch.empty((16, 0), dtype=torch.bfloat16, device=dev)
    w = torch.empty((24, 0), dtype=torch.bfloat16, device=dev)
    y = torch.full((16, 24), 5.0, device=dev)
    q.nvfp4_bf16_gemm(q.FPROP, x, w, out=y)
    dy = torch.ones((0, 24), dtype=torch.bfloat16, device=dev)
    xx = torch.ones((0, 16), dtype=torch.bfloat16, device=dev)
    dw = torch.full((24, 16), 5.0, device=dev)
    q.nvfp4_bf16_gemm(q.WGRAD, dy, xx, out=dw)
    torch.cuda.synchronize()
    assert (y == 0).all().item() and (dw == 0).all().item()
    # empty output: nothing to do
    z = q.nvfp4_bf16_gemm(q.FPROP, torch.empty((0, 32), dtype=torch.bfloat16, device=dev),
                          torch.ones((8, 32), dtype=torch.bfloat16, device=dev))
    assert z.shape == (0, 8)


def test_bf16_gemm_deterministic(env):
    torch, oracle, q, wl, dev = env
    a, b = _operands(wl, 2, 520, 264, 776, 5)
    A, B = to_dev(a, dev), to_dev(b, dev)
    r1 = q.nvfp4_bf16_gemm(q.WGRAD, A, B, torch.float32)
    r2 = q.nvfp4_bf16_gemm(q.WGRAD, A, B, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)


def test_bf16_gemm_rejects_bad_shapes(env):
    torch, oracle, q, wl, dev = env
    x = torch.ones((12, 16), dtype=torch.bfloat16, device=dev)   # M not a multiple of 8
    w = torch.ones((8, 16), dtype=torch.bfloat16, device=dev)
    with pytest.raises(RuntimeError, match="invalid shape"):
        q.nvfp4_bf16_gemm(q.FPROP, x, w)
