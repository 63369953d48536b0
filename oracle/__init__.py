"""CPU oracle for the NVFP4 quantize -> GEMM path.

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and the bench's
cpu_baseline leg may import this package; the product path never does.

Quantisers and codecs come from ``nvfp4_oracle.c`` (fp32, element by
element, no FMA contraction).  The GEMM reference is written here in numpy:
the fp64 product of the two dequantised operands, which is the plain
definition of a GEMM over NVFP4 tensors.

Sources: web pages about NVIDIA's report "Pretraining Large Language Models
with NVFP4" -- the gist.science summary "Pretraining Large Language Models
with NVFP4" (sections "Das Wesentliche", "Technische Zusammenfassung") and
"LLM-Pretraining in 4-Bit: NVIDIA stellt NVFP4-Trainingsansatz vor".

Parity status: every function here is pinned by tests/test_oracle_*.py to
something other than itself (brute force, exact rationals, closed forms, a
library Philox); none is "parity unpinned".
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("NVFP4_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

BLOCK_1X16 = 0
BLOCK_16X16 = 1
BLOCK_MX32 = 2     # MXFP4: 32-element blocks, UE8M0 scales, no tensor scale
MX_ROWS = 0        # MXFP4 layouts: blocks along the rows of x
MX_COLS = 1        # the transposed matrix, blocks along the columns of x
MX_COLS_RHT = 2    # as MX_COLS after the 16-point RHT of each 16-row chunk
RNE = 0
SR = 1

FPROP = 0
DGRAD = 1
WGRAD = 2

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        u64 = ctypes.c_uint64
        u32 = ctypes.c_uint32
        L.orc_quantize.argtypes = [P, i64, i64, ctypes.c_int, ctypes.c_int, u64, u64, P, P, P, P, P]
        L.orc_quantize.restype = ctypes.c_int
        L.orc_rht_quantize.argtypes = [P, i64, i64, u32, ctypes.c_int, u64, u64, P, P, P, P, P]
        L.orc_rht_quantize.restype = ctypes.c_int
        L.orc_rht_transform.argtypes = [P, i64, i64, u32, P]
        L.orc_rht_transform.restype = ctypes.c_int
        L.orc_rht16.argtypes = [P, u32, P]
        L.orc_rht16.restype = None
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_philox4x32_10.restype = None
        L.orc_sr_draw.argtypes = [u64, u64]
        L.orc_sr_draw.restype = ctypes.c_uint16
        L.orc_sr_draw_n.argtypes = [u64, u64, i64, P]
        L.orc_sr_draw_n.restype = None
        L.orc_rht_sign_mask.argtypes = [u64]
        L.orc_rht_sign_mask.restype = u32
        L.orc_tensor_scale.argtypes = [ctypes.c_float]
        L.orc_tensor_scale.restype = ctypes.c_float
        L.orc_block_scale.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_block_scale.restype = ctypes.c_uint8
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode.restype = ctypes.c_float
        L.orc_e2m1_encode_rne_n.argtypes = [P, i64, P]
        L.orc_e2m1_encode_rne_n.restype = None
        L.orc_e2m1_encode_sr_n.argtypes = [P, P, i64, P]
        L.orc_e2m1_encode_sr_n.restype = None
        L.orc_e4m3_encode_n.argtypes = [P, i64, P]
        L.orc_e4m3_encode_n.restype = None
        L.orc_gemm_fp32.argtypes = [P, P, ctypes.c_int, ctypes.c_float, P, P, ctypes.c_int,
                                    ctypes.c_float, i64, i64, i64, P]
        L.orc_gemm_fp32.restype = ctypes.c_int
        L.orc_rht_signs64.argtypes = [u64]
        L.orc_rht_signs64.restype = u64
        L.orc_rht_sized.argtypes = [P, ctypes.c_int, u64, P]
        L.orc_rht_sized.restype = None
        L.orc_rht_quantize_sized.argtypes = [P, i64, i64, ctypes.c_int, u64, ctypes.c_int, u64, P, P, P, P, P]
        L.orc_rht_quantize_sized.restype = ctypes.c_int
        L.orc_quantize_rht_rows.argtypes = [P, i64, i64, ctypes.c_int, u32, ctypes.c_int, u64, P, P, P, P, P]
        L.orc_quantize_rht_rows.restype = ctypes.c_int
        L.orc_mx_quantize.argtypes = [P, i64, i64, ctypes.c_int, u32, ctypes.c_int, u64, P, P]
        L.orc_mx_quantize.restype = ctypes.c_int
        L.orc_mx_exponent.argtypes = [ctypes.c_float]
        L.orc_mx_exponent.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _u16(x):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as their uint16 bit patterns")
    return x


# ---------------------------------------------------------------------------
# Codecs (array forms)
# ---------------------------------------------------------------------------

def e2m1_encode_rne(y):
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().orc_e2m1_encode_rne_n(_ptr(y), y.size, _ptr(out))
    return out


def e2m1_encode_sr(y, u16):
    y = np.ascontiguousarray(y, dtype=np.float32)
    u = np.ascontiguousarray(u16, dtype=np.uint16)
    assert u.shape == y.shape
    out = np.empty(y.shape, np.uint8)
    lib().orc_e2m1_encode_sr_n(_ptr(y), _ptr(u), y.size, _ptr(out))
    return out


def e4m3_encode(t):
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, np.uint8)
    lib().orc_e4m3_encode_n(_ptr(t), t.size, _ptr(out))
    return out


def e2m1_decode(code):
    return lib().orc_e2m1_decode(int(code))


def e4m3_decode(b):
    return lib().orc_e4m3_decode(int(b))


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    o = np.empty(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return o


def sr_draws(seed, idx0, n):
    out = np.empty(n, np.uint16)
    lib().orc_sr_draw_n(seed, idx0, n, _ptr(out))
    return out


def rht_sign_mask(seed):
    return int(lib().orc_rht_sign_mask(seed))


def tensor_scale(amax):
    return float(lib().orc_tensor_scale(amax))


def block_scale(amax_b, s_enc):
    return int(lib().orc_block_scale(amax_b, s_enc))


def rht16(v, sign_mask):
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.shape == (16,)
    out = np.empty(16, np.float32)
    lib().orc_rht16(_ptr(v), sign_mask, _ptr(out))
    return out


# ---------------------------------------------------------------------------
# Quantisers
# ---------------------------------------------------------------------------

class QTensor:
    """Oracle NVFP4 tensor: tight layouts, numpy arrays."""

    def __init__(self, codes, scales, amax, s_enc, rows, cols, block):
        self.codes = codes      # uint8 rows x cols/2
        self.scales = scales    # uint8 rows x cols/16 (1x16) or rows/16 x cols/16
        self.amax = amax        # float (fp32 value)
        self.s_enc = s_enc      # float (fp32 value)
        self.rows = rows
        self.cols = cols
        self.block = block


def quantize(x_u16, block=BLOCK_1X16, rounding=RNE, seed=0, amax_in=None, idx0=0):
    """NVFP4-quantise a row-major bf16 matrix given as uint16 bits.

    idx0 offsets the stochastic-rounding draw index: rows r0.. of a larger
    tensor, quantised with its amax and idx0 = r0 * cols, give exactly those
    rows of the whole tensor's result.
    """
    x = _u16(x_u16)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    sr = rows if block == BLOCK_1X16 else rows // 16
    scales = np.zeros((sr, cols // 16), np.uint8)
    amax = np.zeros(1, np.float32)
    s_enc = np.zeros(1, np.float32)
    ain = None if amax_in is None else np.array([amax_in], np.float32)
    rc = lib().orc_quantize(_ptr(x), rows, cols, block, rounding, seed, idx0, _ptr(ain), _ptr(codes),
                            _ptr(scales), _ptr(amax), _ptr(s_enc))
    if rc != 0:
        raise ValueError(f"orc_quantize: status {rc}")
    return QTensor(codes, scales, float(amax[0]), float(s_enc[0]), rows, cols, block)


def rht_quantize(x_u16, sign_mask, rounding=RNE, seed=0, amax_in=None, idx0=0):
    """Wgrad operand: RHT along tokens, transpose to channels x tokens, 1x16 quantise.

    idx0 offsets the stochastic-rounding draw index (channels c0.. of a larger
    tensor: idx0 = c0 * tokens, with that tensor's transformed amax).
    """
    x = _u16(x_u16)
    tokens, channels = x.shape
    codes = np.zeros((channels, tokens // 2), np.uint8)
    scales = np.zeros((channels, tokens // 16), np.uint8)
    amax = np.zeros(1, np.float32)
    s_enc = np.zeros(1, np.float32)
    ain = None if amax_in is None else np.array([amax_in], np.float32)
    rc = lib().orc_rht_quantize(_ptr(x), tokens, channels, sign_mask, rounding, seed, idx0, _ptr(ain),
                                _ptr(codes), _ptr(scales), _ptr(amax), _ptr(s_enc))
    if rc != 0:
        raise ValueError(f"orc_rht_quantize: status {rc}")
    return QTensor(codes, scales, float(amax[0]), float(s_enc[0]), channels, tokens, BLOCK_1X16)


def mx_exponent(amax_b):
    """Shared exponent of an MXFP4 block with max |x| = amax_b."""
    return int(lib().orc_mx_exponent(amax_b))


def mx_quantize(x_u16, mode=MX_ROWS, sign_mask=0, rounding=RNE, seed=0):
    """MXFP4 quantisation (the format NVFP4 is compared with, Technische
    Zusammenfassung 2.A): E2M1 codes, one UE8M0 scale per 32 elements.

    mode MX_ROWS: blocks along the rows of x, result rows x cols;
    MX_COLS: the transposed matrix (blocks along the columns of x), result
    cols x rows; MX_COLS_RHT: MX_COLS after the 16-point RHT of every
    16-row chunk of each column (2.B.2).  SR draws are indexed in the
    result's layout.  Returns a QTensor with block BLOCK_MX32 (amax and
    s_enc are None: MXFP4 has no tensor scale).
    """
    x = _u16(x_u16)
    rows, cols = x.shape
    orows, ocols = (rows, cols) if mode == MX_ROWS else (cols, rows)
    codes = np.zeros((orows, ocols // 2), np.uint8)
    scales = np.zeros((orows, ocols // 32), np.uint8)
    rc = lib().orc_mx_quantize(_ptr(x), rows, cols, mode, sign_mask, rounding, seed, _ptr(codes),
                               _ptr(scales))
    if rc != 0:
        raise ValueError(f"orc_mx_quantize: status {rc}")
    return QTensor(codes, scales, None, None, orows, ocols, BLOCK_MX32)


def rht_signs64(seed):
    """64 random signs (bit i: d_i = -1); the low 16 are rht_sign_mask(seed)."""
    return int(lib().orc_rht_signs64(seed))


def rht_sized(v, size, signs):
    """The size-point transform (size 4, 16 or 64) of one fp32 vector."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.shape == (size,)
    out = np.empty(size, np.float32)
    lib().orc_rht_sized(_ptr(v), size, signs, _ptr(out))
    return out


def rht_quantize_sized(x_u16, size, signs, rounding=RNE, seed=0, amax_in=None):
    """Wgrad operand with a size-point RHT along tokens (size 4, 16 or 64;
    the ablation of Technische Zusammenfassung 2.B.2's 16 x 16 choice), then
    transpose and 1x16 quantisation as in rht_quantize."""
    x = _u16(x_u16)
    tokens, channels = x.shape
    codes = np.zeros((channels, tokens // 2), np.uint8)
    scales = np.zeros((channels, tokens // 16), np.uint8)
    amax = np.zeros(1, np.float32)
    s_enc = np.zeros(1, np.float32)
    ain = None if amax_in is None else np.array([amax_in], np.float32)
    rc = lib().orc_rht_quantize_sized(_ptr(x), tokens, channels, size, signs, rounding, seed, _ptr(ain),
                                      _ptr(codes), _ptr(scales), _ptr(amax), _ptr(s_enc))
    if rc != 0:
        raise ValueError(f"orc_rht_quantize_sized: status {rc}")
    return QTensor(codes, scales, float(amax[0]), float(s_enc[0]), channels, tokens, BLOCK_1X16)


def quantize_rht_rows(x_u16, sign_mask, block=BLOCK_1X16, rounding=RNE, seed=0, amax_in=None):
    """The fprop / dgrad operand with the 16-point RHT along its rows (the
    contraction dimension), then NVFP4 quantisation as quantize(); the
    ablation of Technische Zusammenfassung 2.B.2's wgrad-only choice."""
    x = _u16(x_u16)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    sr = rows if block == BLOCK_1X16 else rows // 16
    scales = np.zeros((sr, cols // 16), np.uint8)
    amax = np.zeros(1, np.float32)
    s_enc = np.zeros(1, np.float32)
    ain = None if amax_in is None else np.array([amax_in], np.float32)
    rc = lib().orc_quantize_rht_rows(_ptr(x), rows, cols, block, sign_mask, rounding, seed, _ptr(ain),
                                     _ptr(codes), _ptr(scales), _ptr(amax), _ptr(s_enc))
    if rc != 0:
        raise ValueError(f"orc_quantize_rht_rows: status {rc}")
    return QTensor(codes, scales, float(amax[0]), float(s_enc[0]), rows, cols, block)


def rht_transform(x_u16, sign_mask):
    """fp32 channels x tokens transform of a tokens x channels bf16 matrix."""
    x = _u16(x_u16)
    tokens, channels = x.shape
    out = np.empty((channels, tokens), np.float32)
    rc = lib().orc_rht_transform(_ptr(x), tokens, channels, sign_mask, _ptr(out))
    if rc != 0:
        raise ValueError(f"orc_rht_transform: status {rc}")
    return out


def amax(x_u16, rows_per_chunk=1024):
    """Tensor amax max |x| of a bf16 matrix (the input of the FP32 tensor
    scale, Technische Zusammenfassung 2.A), a slice of rows at a time."""
    x = np.atleast_2d(_u16(x_u16))
    m = 0.0
    for r0 in range(0, x.shape[0], rows_per_chunk):
        v = bf16_bits_to_f64(x[r0:r0 + rows_per_chunk])
        if v.size:
            m = max(m, float(np.abs(v).max()))
    return m


def rht_amax(x_u16, sign_mask, channels_per_chunk=1024):
    """max |RHT(x)| over the whole tokens x channels matrix, evaluated a slice
    of channels at a time (the transform acts on each channel separately)."""
    x = _u16(x_u16)
    tokens, channels = x.shape
    m = 0.0
    for c0 in range(0, channels, channels_per_chunk):
        t = rht_transform(np.ascontiguousarray(x[:, c0:c0 + channels_per_chunk]), sign_mask)
        if t.size:
            m = max(m, float(np.abs(t).max()))
    return m


# ---------------------------------------------------------------------------
# Dequantisation and the GEMM reference (fp64)
# ---------------------------------------------------------------------------

def _e2m1_table():
    # E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa; exponent 0 is subnormal.
    t = np.zeros(16, np.float64)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        t[c] = -mag if s else mag
    return t


def _e4m3_table():
    # OCP E4M3: bias 7, subnormals m * 2^-9, 0x7F/0xFF NaN.
    t = np.zeros(256, np.float64)
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            t[b] = np.nan
            continue
        mag = m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8)
        t[b] = -mag if s else mag
    return t


E2M1_VALUES = _e2m1_table()
E4M3_VALUES = _e4m3_table()


def unpack_codes(codes, cols):
    """uint8 rows x cols/2 -> uint8 rows x cols (one code per element)."""
    lo = codes & 0x0F
    hi = codes >> 4
    out = np.empty((codes.shape[0], cols), np.uint8)
    out[:, 0::2] = lo[:, : cols // 2]
    out[:, 1::2] = hi[:, : cols // 2]
    return out


def dequantize_qs(q: QTensor):
    """Exact q * S_b (fp64) -- the decoded value before the 1/s_enc factor."""
    codes = unpack_codes(q.codes, q.cols)
    vals = E2M1_VALUES[codes]
    S = E4M3_VALUES[q.scales]
    if q.block == BLOCK_1X16:
        S = np.repeat(S, 16, axis=1)
    else:
        S = np.repeat(np.repeat(S, 16, axis=0), 16, axis=1)
    return vals * S


def mx_dequantize(q: QTensor):
    """x^ = q * 2^(scale - 127) (fp64) of an MXFP4 tensor."""
    codes = unpack_codes(q.codes, q.cols)
    S = np.ldexp(1.0, q.scales.astype(np.int64) - 127)
    return E2M1_VALUES[codes] * np.repeat(S, 32, axis=1)


def mx_gemm(a: QTensor, b: QTensor, rows=None):
    """fp64 GEMM of dequantised MXFP4 operands, both rows x K:
    C[m, n] = sum_k a^[m, k] b^[n, k].  rows: optional output rows."""
    if rows is not None:
        rows = np.asarray(rows)
        a = QTensor(a.codes[rows], a.scales[rows], None, None, len(rows), a.cols, a.block)
    return mx_dequantize(a) @ mx_dequantize(b).T


def dequantize(q: QTensor):
    """x^ = q * S_b / s_enc in fp64."""
    return dequantize_qs(q) / np.float64(q.s_enc)


def gemm(pass_, a: QTensor, b: QTensor, rows=None):
    """fp64 GEMM of dequantised NVFP4 operands.

    FPROP: a = X (M x K, 1x16), b = W (N x K, 16x16):      Y  = X^ W^T      (M x N)
    DGRAD: a = dY (M x N, 1x16), b = W (N x K, 16x16):     dX = dY^ W^      (M x K)
    WGRAD: a = RHT(dY)^T (N x M), b = RHT(X)^T (K x M):    dW = A^ B^T      (N x K)
    rows: optional index array of output rows to compute (sampled parity).
    Returns float64.
    """
    alpha = (1.0 / np.float64(a.s_enc)) * (1.0 / np.float64(b.s_enc))
    if rows is not None:
        assert a.block == BLOCK_1X16
        rows = np.asarray(rows)
        sub = QTensor(a.codes[rows], a.scales[rows], a.amax, a.s_enc, len(rows), a.cols, a.block)
        A = dequantize_qs(sub)
    else:
        A = dequantize_qs(a)
    B = dequantize_qs(b)
    if pass_ == DGRAD:
        return (A @ B) * alpha
    return (A @ B.T) * alpha


def gemm_fp32_blocks(a: QTensor, b: QTensor):
    """fp32 GEMM that sums exact 16-element block partials in block order,
    both operands rows x K: P_b = sum of the block's 16 products of E2M1
    values (exact), term = P_b * S_a * S_b (exact), acc = RN(acc + term),
    result RN(acc * alpha).  The reference of the FP8-per-block GEMM
    datapath, whose arithmetic is exactly this."""
    M, K = a.rows, a.cols
    N = b.rows
    assert b.cols == K
    c = np.empty((M, N), np.float32)
    rc = lib().orc_gemm_fp32(_ptr(a.codes), _ptr(a.scales), 1 if a.block == BLOCK_1X16 else 16,
                             a.s_enc, _ptr(b.codes), _ptr(b.scales),
                             1 if b.block == BLOCK_1X16 else 16, b.s_enc, M, N, K, _ptr(c))
    if rc != 0:
        raise ValueError(f"orc_gemm_fp32: status {rc}")
    return c


def bf16_gemm(pass_, a_u16, b_u16, rows=None):
    """fp64 GEMM of a linear layer kept in bf16 (Technische Zusammenfassung
    2.B.1: some layers stay BF16; passes as in 2.B.2).  Plain definition of
    each pass over the exact values of the bf16 operands:

    FPROP: a = X (M x K), b = W (N x K):   Y  = X W^T     (M x N)
    DGRAD: a = dY (M x N), b = W (N x K):  dX = dY W      (M x K)
    WGRAD: a = dY (M x N), b = X (M x K):  dW = dY^T X    (N x K)
    rows: optional index array of output rows to compute (sampled parity).
    Returns float64.
    """
    A = bf16_bits_to_f64(a_u16)
    B = bf16_bits_to_f64(b_u16)
    if pass_ == FPROP:
        A = A if rows is None else A[np.asarray(rows)]
        return A @ B.T
    if pass_ == DGRAD:
        A = A if rows is None else A[np.asarray(rows)]
        return A @ B
    if pass_ == WGRAD:
        At = A.T if rows is None else A.T[np.asarray(rows)]
        return At @ B
    raise ValueError(f"unknown pass {pass_}")


def bf16_bits_to_f64(u16):
    u = np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
