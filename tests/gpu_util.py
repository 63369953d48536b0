"""Helpers shared by the GPU parity tests (comparison only, no method arithmetic)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def ensure_built():
    from quantize_precision_gemm_amd import lib_path
    import oracle

    if not os.path.exists(lib_path()):
        from quantize_precision_gemm_amd import build as hip_build
        hip_build.build()
    if not os.path.exists(oracle._LIB_PATH):
        from oracle import build as oracle_build
        oracle_build.build()


def to_dev(u16, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).to(dev).view(torch.bfloat16)


def assert_same_quant(g, o, what, transposed=None):
    """GPU NVFP4Tensor g equals oracle QTensor o bit for bit."""
    ga, gs = np.float32(g.amax.item()), np.float32(g.s_enc.item())
    assert ga.view(np.uint32) == np.float32(o.amax).view(np.uint32), f"{what}: amax {ga} vs {o.amax}"
    assert gs.view(np.uint32) == np.float32(o.s_enc).view(np.uint32), f"{what}: s_enc {gs} vs {o.s_enc}"
    gc = g.codes_host()
    if not np.array_equal(gc, o.codes):
        bad = np.argwhere(gc != o.codes)
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at ({r},{c}): "
                             f"gpu {gc[r, c]:#04x} oracle {o.codes[r, c]:#04x}")
    gsc = g.scales_host()
    if not np.array_equal(gsc, o.scales):
        bad = np.argwhere(gsc != o.scales)
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} scales differ, first at ({r},{c}): "
                             f"gpu {gsc[r, c]:#04x} oracle {o.scales[r, c]:#04x}")
    if transposed is not None:
        # transposed copy of a 16x16-block tensor equals the oracle's quantisation of W^T
        assert np.array_equal(g.codes_t_host(), transposed.codes), f"{what}: transposed codes"
        assert np.array_equal(g.scales_t_host(), transposed.scales), f"{what}: transposed scales"


def rel_fro(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return np.linalg.norm(got - want) / (den if den > 0 else 1.0)


def bf16_rne_bits(f32):
    """fp32 array -> bf16 bit patterns, round to nearest even (finite values)."""
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)
