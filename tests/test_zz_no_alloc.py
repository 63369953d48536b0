"""nvfp4_gemm_split_noalloc (the entry point for callers that cannot
allocate: its split parts live in a device array inside the library) against
nvfp4_gemm_split with a caller workspace, called through the C ABI.

Passes: "Pretraining Large Language Models with NVFP4" (gist.science
summary), Technische Zusammenfassung 2.B.2.  Both entry points run the same
kernels on the same operands, so the outputs must be identical bit for bit
(a stronger bar than the GEMM's 1e-5 against the oracle, which is also
checked).  Two calls in a row, the second on a smaller problem, then the
first again: the array keeps the previous call's contents, which must not
matter.
"""
import ctypes

import numpy as np
import pytest

from tests.gpu_util import ensure_built, rel_fro, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    ensure_built()
    import oracle
    import quantize_precision_gemm_amd as q
    from quantize_precision_gemm_amd import workloads as wl
    dev = torch.device("cuda:0")
    L = q.load_library()
    D = ctypes.POINTER(q._Desc)
    L.nvfp4_gemm_split_noalloc.argtypes = [ctypes.c_int32, D, D, ctypes.c_void_p, ctypes.c_int64,
                                           ctypes.c_int32, ctypes.c_void_p]
    L.nvfp4_gemm_split_noalloc.restype = ctypes.c_int
    return torch, oracle, q, wl, dev, L


def _problem(env, kind):
    torch, oracle, q, wl, dev, L = env
    rng = np.random.default_rng(7 if kind == "dgrad" else 8)
    if kind == "dgrad":  # dX (1024 x 1280) = dY (1024 x 4096) W (4096 x 1280): 20 tiles
        dy, w = wl.lognormal_rows(rng, (1024, 4096)), wl.normal(rng, (4096, 1280), 0.02)
        a = q.nvfp4_quantize(to_dev(dy, dev), q.BLOCK_1X16, q.SR, 3)
        b = q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16, with_transpose=True)
        want = oracle.gemm(oracle.DGRAD, oracle.quantize(dy, oracle.BLOCK_1X16, oracle.SR, 3),
                           oracle.quantize(w, oracle.BLOCK_16X16))
        return q.DGRAD, a, b, want
    # fprop Y (300 x 528) = X (300 x 4112) W^T: 6 tiles, a K tail
    x, w = wl.student_t_unit_var(rng, (300, 4112), 4), wl.normal(rng, (528, 4112), 0.02)
    a, b = q.nvfp4_quantize(to_dev(x, dev)), q.nvfp4_quantize(to_dev(w, dev), q.BLOCK_16X16)
    want = oracle.gemm(oracle.FPROP, oracle.quantize(x), oracle.quantize(w, oracle.BLOCK_16X16))
    return q.FPROP, a, b, want


def _run(env, kind):
    torch, oracle, q, wl, dev, L = env
    P, a, b, want = _problem(env, kind)
    need = q.nvfp4_gemm_split_workspace(P, a, b)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    if cus > 1:
        assert need > 0  # the split (scratch) path runs
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    for dt, code in ((torch.float32, q.OUT_FP32), (torch.bfloat16, q.OUT_BF16)):
        M, N = want.shape
        got = torch.full((M, N), 3.0, dtype=dt, device=dev)
        da, db = a.descriptor(), b.descriptor()
        print(f"noalloc {kind} {dt}", flush=True)
        st = L.nvfp4_gemm_split_noalloc(P, ctypes.byref(da), ctypes.byref(db), got.data_ptr(),
                                        got.stride(0), code, s)
        assert st == 0, st
        ref = q.nvfp4_gemm_split(P, a, b, ws, out_dtype=dt)
        torch.cuda.synchronize()
        iv = torch.int32 if dt == torch.float32 else torch.int16
        assert torch.equal(got.view(iv), ref.view(iv)), f"{kind} {dt}: differs from nvfp4_gemm_split"
        if dt == torch.float32:
            err = rel_fro(got.cpu().numpy(), want)
            assert err <= 1e-5, f"{kind}: relative Frobenius error {err:.3e}"


def test_noalloc_matches_workspace_entry_point(env):
    _run(env, "dgrad")   # 20 tiles x 8 parts: 40 MiB of the array
    _run(env, "fprop")   # then a smaller problem: 6 tiles x 8 parts, 12 MiB
    _run(env, "dgrad")   # and the first again over the second's leftovers


def test_noalloc_validates_like_the_workspace_entry_point(env):
    torch, oracle, q, wl, dev, L = env
    P, a, b, want = _problem(env, "fprop")
    c = torch.full(want.shape, 5.0, dtype=torch.float32, device=dev)
    da, db = a.descriptor(), b.descriptor()
    s = torch.cuda.current_stream().cuda_stream
    assert L.nvfp4_gemm_split_noalloc(P, ctypes.byref(da), ctypes.byref(db), c.data_ptr(),
                                      c.stride(0), 7, s) == -4  # unknown output dtype
    assert L.nvfp4_gemm_split_noalloc(9, ctypes.byref(da), ctypes.byref(db), c.data_ptr(),
                                      c.stride(0), q.OUT_FP32, s) == -4  # unknown pass
    assert L.nvfp4_gemm_split_noalloc(P, ctypes.byref(da), ctypes.byref(db), None,
                                      c.stride(0), q.OUT_FP32, s) == -1
    torch.cuda.synchronize()
    assert (c == 5.0).all().item()
