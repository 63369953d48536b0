"""Host-side checks of caller-supplied buffers in the Python binding.

The C descriptor (include/nvfp4.h) carries leading dimensions but no buffer
sizes, so a buffer too small for the call can only be caught by the binding,
before anything is launched.  These tests run the checks on CPU tensors (no
GPU needed): each mismatched buffer raises, each well-sized one passes.
"""
import pytest
import torch

import quantize_precision_gemm_amd as q

CPU = torch.device("cpu")


def _nv(rows, cols, block=q.BLOCK_1X16, transpose=False, srows=None, crows=None):
    """An NVFP4Tensor of CPU buffers laid out like alloc_nvfp4's (optionally with
    fewer code or scale rows than the tensor needs)."""
    ld_c = (cols + 31) // 32 * 32 // 2
    per = 32 if block == q.BLOCK_MX32 else 16
    ld_s = max((cols // per + 3) // 4 * 4, 4)
    need_s = rows // 16 if block == q.BLOCK_16X16 else rows
    codes = torch.empty((rows if crows is None else crows, ld_c), dtype=torch.uint8)
    scales = torch.empty((need_s if srows is None else srows, ld_s), dtype=torch.uint8)
    ct = st = None
    if transpose:
        ct = torch.empty((cols, (rows + 31) // 32 * 32 // 2), dtype=torch.uint8)
        st = torch.empty((cols // 16, max((rows // 16 + 3) // 4 * 4, 4)), dtype=torch.uint8)
    return q.NVFP4Tensor(codes, scales, torch.empty(1), torch.empty(1), rows, cols, block, ct, st)


def test_well_sized_buffers_pass():
    q._check_nvfp4_buffers(_nv(64, 96), 64, 96, q.BLOCK_1X16, CPU)
    q._check_nvfp4_buffers(_nv(64, 96, q.BLOCK_16X16, True), 64, 96, q.BLOCK_16X16, CPU, True)
    q._check_nvfp4_buffers(_nv(64, 96, q.BLOCK_MX32), 64, 96, q.BLOCK_MX32, CPU)
    q._check_nvfp4_buffers(_nv(0, 32), 0, 32, q.BLOCK_1X16, CPU)
    q._check_gemm_out(torch.empty(8, 16), (8, 16), CPU)
    wide = torch.empty(8, 40, dtype=torch.bfloat16)
    q._check_gemm_out(wide[:, :16], (8, 16), CPU)  # padded leading dimension


def test_2d_buffer_reused_for_1x16_quantise_raises():
    # the case of a 16x16-block buffer (rows/16 scale rows) reused for a 1x16
    # quantisation: the kernel would write 16x past the scales' end
    out = _nv(64, 96, q.BLOCK_16X16)
    with pytest.raises(ValueError, match="scales"):
        q._check_nvfp4_buffers(out, 64, 96, q.BLOCK_1X16, CPU)


@pytest.mark.parametrize("kind", ["codes_rows", "codes_cols", "scales_rows", "transpose_missing",
                                  "transpose_small", "dtype", "noncontig", "amax"])
def test_undersized_or_wrong_buffers_raise(kind):
    rows, cols = 64, 96
    block = q.BLOCK_16X16 if kind.startswith("transpose") else q.BLOCK_1X16
    t = _nv(rows, cols, block, transpose=kind == "transpose_small")
    if kind == "codes_rows":
        t.codes = torch.empty((rows - 1, t.codes.shape[1]), dtype=torch.uint8)
    elif kind == "codes_cols":
        t.codes = torch.empty((rows, t.codes.shape[1] - 16), dtype=torch.uint8)
    elif kind == "scales_rows":
        t.scales = torch.empty((rows // 2, t.scales.shape[1]), dtype=torch.uint8)
    elif kind == "transpose_small":
        t.codes_t = torch.empty((cols - 16, t.codes_t.shape[1]), dtype=torch.uint8)
    elif kind == "dtype":
        t.codes = torch.empty(t.codes.shape, dtype=torch.int16)
    elif kind == "noncontig":
        t.codes = torch.empty((rows, 2 * t.codes.shape[1]), dtype=torch.uint8)[:, ::2]
    elif kind == "amax":
        t.amax = torch.empty(0)
    with pytest.raises((ValueError, TypeError)):
        q._check_nvfp4_buffers(t, rows, cols, block, CPU, kind.startswith("transpose"))


@pytest.mark.parametrize("shape,dtype", [((8, 15), torch.float32), ((7, 16), torch.float32),
                                         ((8, 16), torch.float16), ((16, 8), torch.bfloat16)])
def test_gemm_output_mismatch_raises(shape, dtype):
    with pytest.raises((ValueError, TypeError)):
        q._check_gemm_out(torch.empty(shape, dtype=dtype), (8, 16), CPU)


def test_gemm_operand_claims_more_rows_than_its_buffers():
    a = _nv(64, 96)
    a.rows = 128  # descriptor says 128 rows, buffers hold 64
    with pytest.raises(ValueError, match="codes"):
        q._check_operand(a, "a")


def test_scalar_outputs():
    q._check_scalar_out(None, "amax_in", CPU)
    q._check_scalar_out(torch.empty(1), "amax_in", CPU)
    with pytest.raises(ValueError):
        q._check_scalar_out(torch.empty(1, dtype=torch.float64), "amax_in", CPU)
    with pytest.raises(ValueError):
        q._check_scalar_out(torch.empty(0), "amax_in", CPU)


@pytest.mark.parametrize("cols", [0, 1, 4, 203, 208])
def test_allocated_gemm_output_pitch(cols):
    # The C ABI takes an output row pitch that is a multiple of 4 elements; the
    # binding's own outputs keep the logical shape and round only the pitch.
    out = q._new_gemm_out((5, cols), torch.bfloat16, CPU)
    assert tuple(out.shape) == (5, cols) and out.dtype == torch.bfloat16
    if cols:
        assert out.stride(1) == 1 and out.stride(0) == (cols + 3) // 4 * 4
    q._check_gemm_out(out, (5, cols), CPU)
