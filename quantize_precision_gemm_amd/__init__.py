"""Python binding of libnvfp4 -- the NVFP4 quantize -> GEMM path for MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libnvfp4.so`` (C ABI in include/nvfp4.h).  PyTorch provides device memory
and the current stream.  There is no CPU fallback: if the library is not
built, every call raises.

Recipe (web pages about NVIDIA's report "Pretraining Large Language Models
with NVFP4", gist.science summary, Technische Zusammenfassung 2.A-2.B):
activations X are quantised 1x16 with round-to-nearest-even, weights W 16x16
with RNE, gradients dY 1x16 with stochastic rounding; the weight-gradient
GEMM gets both inputs through a 16-point random Hadamard transform along the
token dimension.
"""
import ctypes
import os

import torch

__all__ = [
    "BLOCK_1X16", "BLOCK_16X16", "RNE", "SR", "FPROP", "DGRAD", "WGRAD",
    "NVFP4Tensor", "alloc_nvfp4", "nvfp4_quantize", "nvfp4_rht_quantize", "nvfp4_quantize_dual", "nvfp4_gemm",
    "nvfp4_rht_sign_mask", "nvfp4_amax", "nvfp4_bf16_gemm", "nvfp4_mx_quantize",
    "nvfp4_mx_gemm", "nvfp4_rht_quantize_sized", "nvfp4_rht_signs64", "nvfp4_quantize_rht_rows", "BLOCK_MX32", "MX_ROWS", "MX_COLS", "MX_COLS_RHT", "nvfp4_gemm_fp8blk", "nvfp4_gemm_amax", "nvfp4_gemm_split", "nvfp4_gemm_split_workspace", "nvfp4_gemm_split_noalloc",
    "nvfp4_mfma_sustain", "MFMA_SUSTAIN_DECODED", "MFMA_SUSTAIN_RANDOM", "MFMA_SUSTAIN_FP4",
    "LAYOUT_ROW_MAJOR", "LAYOUT_INTERLEAVED", "interleave_codes", "deinterleave_codes",
    "lib_path", "load_library",
]

BLOCK_1X16 = 0
BLOCK_16X16 = 1
BLOCK_MX32 = 2     # MXFP4 comparison format: 32-element blocks, UE8M0 scales
MX_ROWS = 0        # nvfp4_mx_quantize layouts
MX_COLS = 1
MX_COLS_RHT = 2
# Code layouts (nvfp4_tensor.layout): row-major, or code rows interleaved by 4
# in 32-byte pieces, so that one 64-element K step of 4 rows is a 128-byte line.
LAYOUT_ROW_MAJOR = 0
LAYOUT_INTERLEAVED = 1
RNE = 0
SR = 1
FPROP = 0
DGRAD = 1
WGRAD = 2
OUT_BF16 = 0
OUT_FP32 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libnvfp4.so"
_lib = None


def lib_path() -> str:
    """libnvfp4.so next to this file, or the build named by NVFP4_LIB (the
    host-sanitized build of the same sources, for the CPU checks)."""
    return os.environ.get("NVFP4_LIB") or os.path.join(_HERE, _LIB_NAME)


class _Desc(ctypes.Structure):
    """Mirror of struct nvfp4_tensor."""
    _fields_ = [
        ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
        ("codes_t", ctypes.c_void_p), ("scales_t", ctypes.c_void_p),
        ("amax", ctypes.c_void_p), ("s_enc", ctypes.c_void_p),
        ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("ld_codes", ctypes.c_int64), ("ld_scales", ctypes.c_int64),
        ("ld_codes_t", ctypes.c_int64), ("ld_scales_t", ctypes.c_int64),
        ("block", ctypes.c_int32), ("layout", ctypes.c_int32),
    ]


def load_library():
    """Load libnvfp4.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "or python quantize_precision_gemm_amd/build.py")
        L = ctypes.CDLL(path)
        P, i64, i32, u32, u64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_uint32, ctypes.c_uint64)
        D = ctypes.POINTER(_Desc)
        L.nvfp4_quantize.argtypes = [P, i64, i64, i64, i32, i32, u64, P, D, P]
        L.nvfp4_quantize.restype = ctypes.c_int
        L.nvfp4_rht_quantize.argtypes = [P, i64, i64, i64, u32, i32, u64, P, D, P]
        L.nvfp4_rht_quantize.restype = ctypes.c_int
        L.nvfp4_quantize_dual.argtypes = [P, i64, i64, i64, u32, i32, u64, u64, P, P, D, D, P]
        L.nvfp4_quantize_dual.restype = ctypes.c_int
        L.nvfp4_mx_quantize.argtypes = [P, i64, i64, i64, i32, u32, i32, u64, D, P]
        L.nvfp4_mx_quantize.restype = ctypes.c_int
        L.nvfp4_mx_gemm.argtypes = [D, D, P, i64, i32, P]
        L.nvfp4_mx_gemm.restype = ctypes.c_int
        L.nvfp4_quantize_rht_rows.argtypes = [P, i64, i64, i64, i32, u32, i32, u64, P, D, P]
        L.nvfp4_quantize_rht_rows.restype = ctypes.c_int
        L.nvfp4_rht_quantize_sized.argtypes = [P, i64, i64, i64, i32, u64, i32, u64, P, D, P]
        L.nvfp4_rht_quantize_sized.restype = ctypes.c_int
        L.nvfp4_rht_signs64.argtypes = [u64]
        L.nvfp4_rht_signs64.restype = u64
        L.nvfp4_gemm.argtypes = [i32, D, D, P, i64, i32, P]
        L.nvfp4_gemm.restype = ctypes.c_int
        L.nvfp4_gemm_fp8blk.argtypes = [i32, D, D, P, i64, i32, P]
        L.nvfp4_gemm_split.argtypes = [i32, D, D, P, i64, i32, P, i64, P]
        L.nvfp4_gemm_split.restype = ctypes.c_int
        L.nvfp4_gemm_split_workspace.argtypes = [i32, D, D, ctypes.POINTER(i64)]
        L.nvfp4_gemm_split_workspace.restype = ctypes.c_int
        L.nvfp4_gemm_split_noalloc.argtypes = [i32, D, D, P, i64, i32, P]
        L.nvfp4_gemm_split_noalloc.restype = ctypes.c_int
        L.nvfp4_gemm_amax.argtypes = [i32, D, D, P, i64, u32, P, P, P]
        L.nvfp4_gemm_amax.restype = ctypes.c_int
        L.nvfp4_gemm_fp8blk.restype = ctypes.c_int
        L.nvfp4_amax.argtypes = [P, i64, i64, i64, u32, P, P, P]
        L.nvfp4_amax.restype = ctypes.c_int
        L.nvfp4_bf16_gemm.argtypes = [i32, P, i64, P, i64, i64, i64, i64, P, i64, i32, P]
        L.nvfp4_bf16_gemm.restype = ctypes.c_int
        L.nvfp4_rht_sign_mask.argtypes = [u64]
        L.nvfp4_rht_sign_mask.restype = u32
        L.nvfp4_mfma_sustain.argtypes = [i64, i64, i32, P, P]
        L.nvfp4_mfma_sustain.restype = ctypes.c_int
        L.nvfp4_status_string.argtypes = [i32]
        L.nvfp4_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status, what):
    if status != 0:
        msg = load_library().nvfp4_status_string(status).decode()
        raise RuntimeError(f"{what} failed: status {status} ({msg})")


def _round_up(v, m):
    return (v + m - 1) // m * m


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class NVFP4Tensor:
    """Device buffers of an NVFP4 tensor (rows x cols, blocks along cols).

    codes  uint8 [rows, ld_codes]     two E2M1 codes per byte, low nibble first;
           row-major, or (layout LAYOUT_INTERLEAVED) [round_up(rows, 4), ld_codes]
           bytes holding the code rows interleaved by 4 (interleave_codes)
    scales uint8 [rows or rows/16, ld_scales]   E4M3 block scales (row-major)
    codes_t / scales_t  (16x16 only, optional) the transposed copy used by dgrad,
           codes_t in the same layout as codes
    amax, s_enc  float32 [1]  tensor amax and FP32 encode scale (device)
    """

    def __init__(self, codes, scales, amax, s_enc, rows, cols, block, codes_t=None,
                 scales_t=None, layout=LAYOUT_ROW_MAJOR):
        self.codes, self.scales, self.amax, self.s_enc = codes, scales, amax, s_enc
        self.codes_t, self.scales_t = codes_t, scales_t
        self.rows, self.cols, self.block = rows, cols, block
        self.layout = layout

    def descriptor(self) -> _Desc:
        d = _Desc()
        d.codes, d.scales = self.codes.data_ptr(), self.scales.data_ptr()
        d.codes_t = self.codes_t.data_ptr() if self.codes_t is not None else None
        d.scales_t = self.scales_t.data_ptr() if self.scales_t is not None else None
        d.amax, d.s_enc = self.amax.data_ptr(), self.s_enc.data_ptr()
        d.rows, d.cols = self.rows, self.cols
        d.ld_codes, d.ld_scales = self.codes.shape[1], self.scales.shape[1]
        d.ld_codes_t = self.codes_t.shape[1] if self.codes_t is not None else 0
        d.ld_scales_t = self.scales_t.shape[1] if self.scales_t is not None else 0
        d.block = self.block
        d.layout = self.layout
        return d

    # --- host copies in the tight row-major layout (for checks) ---
    def codes_host(self):
        c = self.codes.cpu().numpy()
        if self.layout == LAYOUT_INTERLEAVED:
            c = deinterleave_codes(c, self.rows)
        return c[: self.rows, : self.cols // 2]

    def scales_host(self):
        per = 32 if self.block == BLOCK_MX32 else 16
        return self.scales[:, : self.cols // per].cpu().numpy()

    def codes_t_host(self):
        c = self.codes_t.cpu().numpy()
        if self.layout == LAYOUT_INTERLEAVED:
            c = deinterleave_codes(c, self.cols)
        return c[: self.cols, : self.rows // 2]

    def scales_t_host(self):
        return self.scales_t[:, : self.rows // 16].cpu().numpy()


def _code_buf_shape(rows, cols, layout):
    """(buffer rows, ld bytes) of the codes of a rows x cols tensor."""
    if layout == LAYOUT_INTERLEAVED:
        return _round_up(rows, 4), _round_up(cols, 64) // 2
    return rows, _round_up(cols, 32) // 2


def alloc_nvfp4(rows, cols, block=BLOCK_1X16, with_transpose=False, device=None,
                layout=LAYOUT_ROW_MAJOR):
    """Allocate the device buffers of a rows x cols NVFP4 tensor (padded leading dims)."""
    device = device or torch.device("cuda", torch.cuda.current_device())
    if layout not in (LAYOUT_ROW_MAJOR, LAYOUT_INTERLEAVED):
        raise ValueError(f"unknown code layout {layout}")
    if block == BLOCK_MX32 and layout != LAYOUT_ROW_MAJOR:
        raise ValueError("MXFP4 tensors are row-major")
    ld_s = _round_up(max(cols // (32 if block == BLOCK_MX32 else 16), 1), 4)
    srows = rows // 16 if block == BLOCK_16X16 else rows
    codes = torch.empty(_code_buf_shape(rows, cols, layout), dtype=torch.uint8, device=device)
    scales = torch.empty((srows, ld_s), dtype=torch.uint8, device=device)
    amax = torch.empty(1, dtype=torch.float32, device=device)
    s_enc = torch.empty(1, dtype=torch.float32, device=device)
    ct = st = None
    if with_transpose:
        ct = torch.empty(_code_buf_shape(cols, rows, layout), dtype=torch.uint8, device=device)
        st = torch.empty((cols // 16, _round_up(max(rows // 16, 1), 4)), dtype=torch.uint8,
                         device=device)
    return NVFP4Tensor(codes, scales, amax, s_enc, rows, cols, block, ct, st, layout)


def interleave_codes(codes):
    """Row-major code rows (numpy uint8 [rows, ld], ld a multiple of 32) in the
    interleaved layout: [round_up(rows, 4), ld] bytes in which byte j of row r
    lies at flat offset (r // 4) * 4 * ld + (j // 32) * 128 + (r % 4) * 32 + j % 32
    (padding rows zero)."""
    import numpy as np
    rows, ld = codes.shape
    if ld % 32:
        raise ValueError("interleaved code rows are a multiple of 32 bytes")
    pad = np.zeros((_round_up(rows, 4), ld), dtype=np.uint8)
    pad[:rows] = codes
    g = pad.reshape(-1, 4, ld // 32, 32).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(g).reshape(-1, ld)


def deinterleave_codes(buf, rows):
    """The inverse of interleave_codes: the first `rows` code rows, row-major."""
    import numpy as np
    n, ld = buf.shape
    if n % 4 or ld % 32:
        raise ValueError("an interleaved codes buffer has whole 4-row groups of 32-byte pieces")
    g = np.ascontiguousarray(buf).reshape(-1, ld // 32, 4, 32).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(g).reshape(-1, ld)[:rows]


def _check_bf16(x):
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 2):
        raise TypeError("expected a 2-D bfloat16 CUDA tensor")
    if x.stride(1) != 1:
        raise ValueError("the last dimension must be contiguous")


def _check_buf(t, what, device, dtype, min_shape):
    """A caller-supplied buffer: a 2-D (or, for min_shape of length 1, 1-D)
    contiguous tensor of `dtype` on `device`, at least `min_shape` large.
    The C descriptor carries no buffer sizes, so this is the only place an
    undersized buffer can be caught before a kernel writes past its end."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{what}: on {t.device}, expected {device}")
    if t.dim() != len(min_shape):
        raise ValueError(f"{what}: {t.dim()}-D, expected {len(min_shape)}-D")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous (its row length is its leading dimension)")
    if any(have < need for have, need in zip(t.shape, min_shape)):
        raise ValueError(f"{what}: shape {tuple(t.shape)} smaller than the {tuple(min_shape)} needed")


def _same_device(a, b):
    """torch devices compare unequal for cuda vs cuda:0; normalise the index."""
    if a.type != b.type:
        return False
    ia = a.index if a.index is not None else (torch.cuda.current_device() if a.type == "cuda" else None)
    ib = b.index if b.index is not None else (torch.cuda.current_device() if b.type == "cuda" else None)
    return ia == ib


def _check_nvfp4_buffers(t, rows, cols, block, device, with_transpose=False, what="out"):
    """Every buffer of an NVFP4 (or MXFP4) tensor is large enough for a
    rows x cols tensor with `block` layout, on `device`."""
    if not isinstance(t, NVFP4Tensor):
        raise TypeError(f"{what}: expected an NVFP4Tensor")
    device = t.codes.device if device is None else device
    if not _same_device(t.codes.device, device):
        raise ValueError(f"{what}.codes: on {t.codes.device}, expected {device}")
    device = t.codes.device
    per = 32 if block == BLOCK_MX32 else 16
    srows = rows // 16 if block == BLOCK_16X16 else rows
    layout = getattr(t, "layout", LAYOUT_ROW_MAJOR)
    if layout not in (LAYOUT_ROW_MAJOR, LAYOUT_INTERLEAVED):
        raise ValueError(f"{what}: unknown code layout {layout}")
    if block == BLOCK_MX32 and layout != LAYOUT_ROW_MAJOR:
        raise ValueError(f"{what}: MXFP4 tensors are row-major")
    il = layout == LAYOUT_INTERLEAVED
    if il and t.codes.dim() == 2 and t.codes.shape[1] % 32:
        raise ValueError(f"{what}.codes: interleaved code rows must be a multiple of 32 bytes")
    _check_buf(t.codes, f"{what}.codes", device, torch.uint8,
               (_round_up(rows, 4) if il else rows, _round_up(cols, 32) // 2))
    _check_buf(t.scales, f"{what}.scales", device, torch.uint8, (srows, cols // per))
    if block != BLOCK_MX32:
        _check_buf(t.amax, f"{what}.amax", device, torch.float32, (1,))
        _check_buf(t.s_enc, f"{what}.s_enc", device, torch.float32, (1,))
    if with_transpose:
        if t.codes_t is None or t.scales_t is None:
            raise ValueError(f"{what}: the transposed copy was asked for but has no buffers")
        if il and t.codes_t.dim() == 2 and t.codes_t.shape[1] % 32:
            raise ValueError(f"{what}.codes_t: interleaved code rows must be a multiple of 32 bytes")
        _check_buf(t.codes_t, f"{what}.codes_t", device, torch.uint8,
                   (_round_up(cols, 4) if il else cols, _round_up(rows, 32) // 2))
        _check_buf(t.scales_t, f"{what}.scales_t", device, torch.uint8, (cols // 16, rows // 16))


def _check_operand(t, what):
    """A GEMM operand: its buffers hold what its descriptor claims."""
    _check_nvfp4_buffers(t, t.rows, t.cols, t.block, None, False, what)


def _check_gemm_out(out, shape, device, dtypes=(torch.float32, torch.bfloat16)):
    if not isinstance(out, torch.Tensor):
        raise TypeError("out: expected a tensor")
    if out.dtype not in dtypes:
        raise TypeError(f"output must be one of {dtypes} with a contiguous last dimension")
    if out.dim() != 2 or tuple(out.shape) != tuple(shape):
        raise ValueError(f"out: shape {tuple(out.shape)}, expected {tuple(shape)}")
    if out.numel() > 0 and out.stride(1) != 1:
        raise TypeError("output must have a contiguous last dimension")
    if out.numel() > 0 and out.stride(0) < shape[1]:
        raise ValueError("out: row stride shorter than a row")
    if not _same_device(out.device, device):
        raise ValueError(f"out: on {out.device}, expected {device}")


def _new_gemm_out(shape, dtype, device):
    """A GEMM output of `shape`: row pitch rounded up to 4 elements (the ABI's
    ldc % 4 rule), so the result is a [:, :cols] view when cols % 4 != 0."""
    rows, cols = shape
    if cols % 4 == 0:
        return torch.empty(shape, dtype=dtype, device=device)
    return torch.empty((rows, _round_up(cols, 4)), dtype=dtype, device=device)[:, :cols]


def _check_scalar_out(t, what, device):
    if t is not None:
        _check_buf(t, what, device, torch.float32, (1,))


def nvfp4_quantize(x, block=BLOCK_1X16, rounding=RNE, seed=0, amax_in=None,
                   with_transpose=False, out=None, layout=LAYOUT_ROW_MAJOR, stream=None):
    """Quantise a row-major bf16 matrix to NVFP4 (see nvfp4_quantize in nvfp4.h)."""
    _check_bf16(x)
    rows, cols = x.shape
    if out is None:
        out = alloc_nvfp4(rows, cols, block, with_transpose and block == BLOCK_16X16, x.device,
                          layout)
    _check_nvfp4_buffers(out, rows, cols, block, x.device,
                         out.codes_t is not None or out.scales_t is not None)
    _check_scalar_out(amax_in, "amax_in", x.device)
    d = out.descriptor()
    st = load_library().nvfp4_quantize(_ptr(x), rows, cols, x.stride(0), block, rounding,
                                       seed, _ptr(amax_in), ctypes.byref(d), _stream(stream))
    _check(st, "nvfp4_quantize")
    out.rows, out.cols, out.block = d.rows, d.cols, d.block
    return out


def nvfp4_rht_quantize(x, sign_mask, rounding=RNE, seed=0, amax_in=None, out=None,
                       layout=LAYOUT_ROW_MAJOR, stream=None):
    """RHT along tokens + transpose + 1x16 quantisation (see nvfp4_rht_quantize)."""
    _check_bf16(x)
    tokens, channels = x.shape
    if out is None:
        out = alloc_nvfp4(channels, tokens, BLOCK_1X16, False, x.device, layout)
    _check_nvfp4_buffers(out, channels, tokens, BLOCK_1X16, x.device)
    _check_scalar_out(amax_in, "amax_in", x.device)
    d = out.descriptor()
    st = load_library().nvfp4_rht_quantize(_ptr(x), tokens, channels, x.stride(0), sign_mask,
                                           rounding, seed, _ptr(amax_in), ctypes.byref(d),
                                           _stream(stream))
    _check(st, "nvfp4_rht_quantize")
    out.rows, out.cols, out.block = d.rows, d.cols, d.block
    return out


def nvfp4_quantize_dual(x, sign_mask, rounding=RNE, seed=0, seed_rht=0, amax_in=None,
                        amax_rht_in=None, out=None, out_rht=None, layout=LAYOUT_ROW_MAJOR,
                        stream=None):
    """Both operands of one tensor from one read (see nvfp4_quantize_dual).

    Returns (the 1x16 tokens x channels operand, the RHT-transposed
    channels x tokens operand)."""
    _check_bf16(x)
    tokens, channels = x.shape
    if out is None:
        out = alloc_nvfp4(tokens, channels, BLOCK_1X16, False, x.device, layout)
    if out_rht is None:
        out_rht = alloc_nvfp4(channels, tokens, BLOCK_1X16, False, x.device, layout)
    _check_nvfp4_buffers(out, tokens, channels, BLOCK_1X16, x.device)
    _check_nvfp4_buffers(out_rht, channels, tokens, BLOCK_1X16, x.device, what="out_rht")
    _check_scalar_out(amax_in, "amax_in", x.device)
    _check_scalar_out(amax_rht_in, "amax_rht_in", x.device)
    d, dr = out.descriptor(), out_rht.descriptor()
    ld_x = x.stride(0) if channels > 0 else 0  # no row stride without columns
    st = load_library().nvfp4_quantize_dual(_ptr(x), tokens, channels, ld_x, sign_mask,
                                            rounding, seed, seed_rht, _ptr(amax_in),
                                            _ptr(amax_rht_in), ctypes.byref(d),
                                            ctypes.byref(dr), _stream(stream))
    _check(st, "nvfp4_quantize_dual")
    out.rows, out.cols, out.block = d.rows, d.cols, d.block
    out_rht.rows, out_rht.cols, out_rht.block = dr.rows, dr.cols, dr.block
    return out, out_rht


def nvfp4_quantize_rht_rows(x, sign_mask, block=BLOCK_1X16, rounding=RNE, seed=0, amax_in=None,
                            with_transpose=False, out=None, layout=LAYOUT_ROW_MAJOR, stream=None):
    """nvfp4_quantize after the 16-point RHT along the rows (see
    nvfp4_quantize_rht_rows in nvfp4.h)."""
    _check_bf16(x)
    rows, cols = x.shape
    if out is None:
        out = alloc_nvfp4(rows, cols, block, with_transpose and block == BLOCK_16X16, x.device, layout)
    _check_nvfp4_buffers(out, rows, cols, block, x.device,
                         out.codes_t is not None or out.scales_t is not None)
    _check_scalar_out(amax_in, "amax_in", x.device)
    d = out.descriptor()
    st = load_library().nvfp4_quantize_rht_rows(_ptr(x), rows, cols, x.stride(0), block, sign_mask,
                                                rounding, seed, _ptr(amax_in), ctypes.byref(d),
                                                _stream(stream))
    _check(st, "nvfp4_quantize_rht_rows")
    out.rows, out.cols, out.block = d.rows, d.cols, d.block
    return out


def nvfp4_rht_quantize_sized(x, size, signs, rounding=RNE, seed=0, amax_in=None, out=None,
                             layout=LAYOUT_ROW_MAJOR, stream=None):
    """Wgrad operand with a `size`-token transform: 1 (none), 4, 16 or 64
    (see nvfp4_rht_quantize_sized in nvfp4.h)."""
    _check_bf16(x)
    tokens, channels = x.shape
    if out is None:
        out = alloc_nvfp4(channels, tokens, BLOCK_1X16, False, x.device, layout)
    _check_nvfp4_buffers(out, channels, tokens, BLOCK_1X16, x.device)
    _check_scalar_out(amax_in, "amax_in", x.device)
    d = out.descriptor()
    st = load_library().nvfp4_rht_quantize_sized(_ptr(x), tokens, channels, x.stride(0), size,
                                                 signs, rounding, seed, _ptr(amax_in),
                                                 ctypes.byref(d), _stream(stream))
    _check(st, "nvfp4_rht_quantize_sized")
    out.rows, out.cols, out.block = d.rows, d.cols, d.block
    return out


def nvfp4_rht_signs64(seed):
    """64 random signs drawn from `seed` (the low 16 are nvfp4_rht_sign_mask)."""
    return int(load_library().nvfp4_rht_signs64(seed))


def nvfp4_mx_quantize(x, mode=MX_ROWS, sign_mask=0, rounding=RNE, seed=0, out=None, stream=None):
    """MXFP4 quantisation (see nvfp4_mx_quantize in nvfp4.h); MX_ROWS gives
    rows x cols, MX_COLS / MX_COLS_RHT the transposed cols x rows."""
    _check_bf16(x)
    rows, cols = x.shape
    orows, ocols = (rows, cols) if mode == MX_ROWS else (cols, rows)
    if out is None:
        out = alloc_nvfp4(orows, ocols, BLOCK_MX32, False, x.device)
    _check_nvfp4_buffers(out, orows, ocols, BLOCK_MX32, x.device)
    d = out.descriptor()
    ld_x = x.stride(0) if cols > 0 else 0
    st = load_library().nvfp4_mx_quantize(_ptr(x), rows, cols, ld_x, mode, sign_mask, rounding,
                                          seed, ctypes.byref(d), _stream(stream))
    _check(st, "nvfp4_mx_quantize")
    out.rows, out.cols, out.block = d.rows, d.cols, d.block
    return out


def nvfp4_mx_gemm(a, b, out_dtype=torch.bfloat16, out=None, stream=None):
    """c = a^ b^T over MXFP4 operands (see nvfp4_mx_gemm in nvfp4.h)."""
    M, N = a.rows, b.rows
    _check_operand(a, "a")
    _check_operand(b, "b")
    if out is None:
        out = _new_gemm_out((M, N), out_dtype, a.codes.device)
    _check_gemm_out(out, (M, N), a.codes.device)
    dt = OUT_FP32 if out.dtype == torch.float32 else OUT_BF16
    da, db = a.descriptor(), b.descriptor()
    st = load_library().nvfp4_mx_gemm(ctypes.byref(da), ctypes.byref(db), _ptr(out),
                                      out.stride(0) if N > 0 else 0, dt, _stream(stream))
    _check(st, "nvfp4_mx_gemm")
    return out


def nvfp4_gemm(pass_, a, b, out_dtype=torch.bfloat16, out=None, stream=None, fp8_blocks=False):
    """NVFP4 GEMM for FPROP / DGRAD / WGRAD (see nvfp4_gemm in nvfp4.h).

    fp8_blocks=True runs the second datapath (nvfp4_gemm_fp8blk)."""
    M = a.rows
    N = b.cols if pass_ == DGRAD else b.rows
    _check_operand(a, "a")
    _check_operand(b, "b")
    if pass_ == DGRAD:
        _check_nvfp4_buffers(b, b.rows, b.cols, b.block, a.codes.device, True, "b")
    if out is None:
        out = _new_gemm_out((M, N), out_dtype, a.codes.device)
    _check_gemm_out(out, (M, N), a.codes.device)
    dt = OUT_FP32 if out.dtype == torch.float32 else OUT_BF16
    da, db = a.descriptor(), b.descriptor()
    fn = load_library().nvfp4_gemm_fp8blk if fp8_blocks else load_library().nvfp4_gemm
    st = fn(pass_, ctypes.byref(da), ctypes.byref(db), _ptr(out), out.stride(0), dt,
            _stream(stream))
    _check(st, "nvfp4_gemm_fp8blk" if fp8_blocks else "nvfp4_gemm")
    return out


def nvfp4_gemm_split_workspace(pass_, a, b):
    """Workspace bytes nvfp4_gemm_split needs for this pass and these operands
    on the current device (0: the tiles fill whole waves)."""
    _check_operand(a, "a")
    _check_operand(b, "b")
    n = ctypes.c_int64(0)
    da, db = a.descriptor(), b.descriptor()
    _check(load_library().nvfp4_gemm_split_workspace(pass_, ctypes.byref(da), ctypes.byref(db),
                                                     ctypes.byref(n)), "nvfp4_gemm_split_workspace")
    return int(n.value)


def nvfp4_gemm_split(pass_, a, b, workspace=None, out_dtype=torch.bfloat16, out=None, stream=None):
    """nvfp4_gemm with the last partial wave of tiles split along K into
    `workspace` (a uint8 device tensor of at least nvfp4_gemm_split_workspace
    bytes; allocated here when None) -- see nvfp4_gemm_split in nvfp4.h."""
    M = a.rows
    N = b.cols if pass_ == DGRAD else b.rows
    need = nvfp4_gemm_split_workspace(pass_, a, b)
    if pass_ == DGRAD:
        _check_nvfp4_buffers(b, b.rows, b.cols, b.block, a.codes.device, True, "b")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=a.codes.device)
    if workspace is not None:
        _check_buf(workspace, "workspace", a.codes.device, torch.uint8, (need,))
    if out is None:
        out = _new_gemm_out((M, N), out_dtype, a.codes.device)
    _check_gemm_out(out, (M, N), a.codes.device)
    dt = OUT_FP32 if out.dtype == torch.float32 else OUT_BF16
    da, db = a.descriptor(), b.descriptor()
    st = load_library().nvfp4_gemm_split(pass_, ctypes.byref(da), ctypes.byref(db), _ptr(out),
                                         out.stride(0), dt, _ptr(workspace),
                                         0 if workspace is None else workspace.numel(),
                                         _stream(stream))
    _check(st, "nvfp4_gemm_split")
    return out


def nvfp4_gemm_split_noalloc(pass_, a, b, out_dtype=torch.bfloat16, out=None, stream=None):
    """nvfp4_gemm_split with the library's own device array as its workspace
    (see nvfp4_gemm_split_noalloc in nvfp4.h: nothing is allocated by the
    call when `out` is given; calls that overlap on one GPU race)."""
    M = a.rows
    N = b.cols if pass_ == DGRAD else b.rows
    _check_operand(a, "a")
    _check_operand(b, "b")
    if pass_ == DGRAD:
        _check_nvfp4_buffers(b, b.rows, b.cols, b.block, a.codes.device, True, "b")
    if out is None:
        out = _new_gemm_out((M, N), out_dtype, a.codes.device)
    _check_gemm_out(out, (M, N), a.codes.device)
    dt = OUT_FP32 if out.dtype == torch.float32 else OUT_BF16
    da, db = a.descriptor(), b.descriptor()
    st = load_library().nvfp4_gemm_split_noalloc(pass_, ctypes.byref(da), ctypes.byref(db),
                                                 _ptr(out), out.stride(0), dt, _stream(stream))
    _check(st, "nvfp4_gemm_split_noalloc")
    return out


def nvfp4_gemm_amax(pass_, a, b, sign_mask=0, rht=True, out=None, amax=None, amax_rht=None,
                    stream=None):
    """FPROP / DGRAD GEMM with bf16 output whose epilogue also writes the
    output's tensor amax and, with rht=True, the amax of its 16-point RHT
    along the rows (see nvfp4_gemm_amax in nvfp4.h).

    Returns (c, amax, amax_rht or None); the maxima are one-element float32
    device tensors, ready as amax_in / amax_rht_in of nvfp4_quantize_dual."""
    M = a.rows
    N = b.cols if pass_ == DGRAD else b.rows
    dev = a.codes.device
    _check_operand(a, "a")
    _check_operand(b, "b")
    if pass_ == DGRAD:
        _check_nvfp4_buffers(b, b.rows, b.cols, b.block, dev, True, "b")
    if out is None:
        out = _new_gemm_out((M, N), torch.bfloat16, dev)
    _check_gemm_out(out, (M, N), dev, (torch.bfloat16,))
    _check_scalar_out(amax, "amax", dev)
    _check_scalar_out(amax_rht if rht else None, "amax_rht", dev)
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=dev)
    if rht and amax_rht is None:
        amax_rht = torch.empty(1, dtype=torch.float32, device=dev)
    if not rht:
        amax_rht = None
    da, db = a.descriptor(), b.descriptor()
    st = load_library().nvfp4_gemm_amax(pass_, ctypes.byref(da), ctypes.byref(db), _ptr(out),
                                        out.stride(0), sign_mask, _ptr(amax), _ptr(amax_rht),
                                        _stream(stream))
    _check(st, "nvfp4_gemm_amax")
    return out, amax, amax_rht


def nvfp4_bf16_gemm(pass_, a, b, out_dtype=torch.bfloat16, out=None, stream=None):
    """GEMM of a linear layer kept in bf16 (see nvfp4_bf16_gemm in nvfp4.h).

    FPROP: a = X (M x K), b = W (N x K) -> M x N
    DGRAD: a = dY (M x N), b = W (N x K) -> M x K
    WGRAD: a = dY (M x N), b = X (M x K) -> N x K
    """
    _check_bf16(a)
    _check_bf16(b)
    if pass_ == FPROP:
        (M, K), N = a.shape, b.shape[0]
        shape = (M, N)
    elif pass_ == DGRAD:
        (M, N), K = a.shape, b.shape[1]
        shape = (M, K)
    elif pass_ == WGRAD:
        (M, N), K = a.shape, b.shape[1]
        shape = (N, K)
    else:
        raise ValueError(f"unknown pass {pass_}")
    if out is None:
        out = _new_gemm_out(shape, out_dtype, a.device)
    _check_gemm_out(out, shape, a.device)
    if not _same_device(b.device, a.device):
        raise ValueError(f"b: on {b.device}, expected {a.device}")
    dt = OUT_FP32 if out.dtype == torch.float32 else OUT_BF16
    def ld(t):  # a matrix without columns has no meaningful row stride
        return t.stride(0) if t.shape[1] > 0 else 0
    st = load_library().nvfp4_bf16_gemm(pass_, _ptr(a), ld(a), _ptr(b), ld(b), M, N, K,
                                        _ptr(out), ld(out), dt, _stream(stream))
    _check(st, "nvfp4_bf16_gemm")
    return out


MFMA_SUSTAIN_DECODED, MFMA_SUSTAIN_RANDOM, MFMA_SUSTAIN_FP4 = 0, 1, 2


def nvfp4_mfma_sustain(blocks, iters, operands=MFMA_SUSTAIN_DECODED, out=None, device=None,
                       stream=None):
    """Register-only stream of a GEMM's matrix instruction (see
    nvfp4_mfma_sustain in nvfp4.h), a measurement aid: time it to learn the
    matrix throughput the GPU sustains.  Returns (out, flops of the call)."""
    dev = device if device is not None else (out.device if out is not None else torch.device("cuda"))
    if out is None:
        out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    _check_buf(out, "out", out.device, torch.float32, (blocks * 512,))
    st = load_library().nvfp4_mfma_sustain(blocks, iters, operands, _ptr(out), _stream(stream))
    _check(st, "nvfp4_mfma_sustain")
    k_inst = 64 if operands == MFMA_SUSTAIN_FP4 else 16
    return out, 2.0 * 32 * 32 * k_inst * 64 * 8 * iters * blocks


def nvfp4_amax(x, sign_mask=None, amax=None, amax_rht=None, stream=None):
    """max |x| and, if sign_mask is given, max |RHT(x)| in one pass (see nvfp4_amax).

    Returns (amax, amax_rht) as 1-element float32 device tensors (amax_rht None
    without a sign mask); pass them as amax_in to the quantisers.
    """
    _check_bf16(x)
    rows, cols = x.shape
    _check_scalar_out(amax, "amax", x.device)
    _check_scalar_out(amax_rht if sign_mask is not None else None, "amax_rht", x.device)
    amax = amax if amax is not None else torch.empty(1, dtype=torch.float32, device=x.device)
    if sign_mask is not None and amax_rht is None:
        amax_rht = torch.empty(1, dtype=torch.float32, device=x.device)
    st = load_library().nvfp4_amax(_ptr(x), rows, cols, x.stride(0),
                                   0 if sign_mask is None else sign_mask, _ptr(amax),
                                   _ptr(amax_rht) if sign_mask is not None else None,
                                   _stream(stream))
    _check(st, "nvfp4_amax")
    return amax, (amax_rht if sign_mask is not None else None)


def nvfp4_rht_sign_mask(seed):
    """The 16 random signs of the Hadamard transform drawn from `seed` (bit i: d_i = -1)."""
    return int(load_library().nvfp4_rht_sign_mask(seed))
