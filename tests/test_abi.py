"""The C-ABI library loads and exports every function include/nvfp4.h declares;
host-side argument validation rejects bad calls before anything is enqueued.
CPU only: no compute call is made."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def lib():
    from quantize_precision_gemm_amd import lib_path, load_library
    if not os.path.exists(lib_path()):
        from quantize_precision_gemm_amd import build as hip_build
        hip_build.build()
    return load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ["nvfp4_quantize", "nvfp4_rht_quantize", "nvfp4_gemm", "nvfp4_rht_sign_mask",
              "nvfp4_status_string"]:
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    from quantize_precision_gemm_amd import lib_path
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for st, s in [(0, b"ok"), (-1, b"null pointer"), (-2, b"invalid shape"),
                  (-3, b"misaligned pointer or leading dimension"), (-4, b"unknown mode"),
                  (-5, b"operands inconsistent with the pass"), (-6, b"kernel launch failed"),
                  (-7, b"workspace missing or too small")]:
        assert lib.nvfp4_status_string(st) == s


def test_sign_mask_matches_oracle(lib):
    import oracle
    for seed in [0, 1, 1000, 2 ** 63 + 7]:
        assert lib.nvfp4_rht_sign_mask(seed) == oracle.rht_sign_mask(seed)


def _desc(**kw):
    from quantize_precision_gemm_amd import _Desc
    d = _Desc()
    for k, v in kw.items():
        setattr(d, k, v)
    return d


FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,status", [
    # x, rows, cols, ld_x, block, rounding
    ((FAKE, 16, 17, 32, 0, 0), -2),          # cols not a multiple of 16
    ((FAKE, 8, 32, 32, 1, 0), -2),           # 16x16 needs rows % 16 == 0
    ((FAKE, 16, 32, 32, 2, 0), -4),          # unknown block
    ((FAKE, 16, 32, 32, 0, 5), -4),          # unknown rounding
    ((None, 16, 32, 32, 0, 0), -1),          # null input
    ((FAKE, 16, 32, 16, 0, 0), -2),          # ld_x < cols
    ((FAKE + 2, 16, 32, 32, 0, 0), -3),      # misaligned input
    ((FAKE, 16, 32, 36, 0, 0), -3),          # ld_x not a multiple of 8
    ((FAKE, -1, 32, 32, 0, 0), -2),          # negative rows
])
def test_quantize_validation(lib, args, status):
    x, rows, cols, ld, block, rnd = args
    d = _desc(codes=FAKE, scales=FAKE, amax=FAKE, s_enc=FAKE, ld_codes=16, ld_scales=4)
    st = lib.nvfp4_quantize(x, rows, cols, ld, block, rnd, 0, None, ctypes.byref(d), None)
    assert st == status


@pytest.mark.parametrize("field,value,status", [
    ("codes", None, -1), ("amax", None, -1), ("s_enc", None, -1),
    ("codes", FAKE + 8, -3), ("ld_codes", 8, -3), ("ld_scales", 2, -3), ("ld_codes", 0, -2),
    ("codes_t", FAKE, -4),   # transposed copy only for 16x16 blocks
])
def test_quantize_out_validation(lib, field, value, status):
    d = _desc(codes=FAKE, scales=FAKE, amax=FAKE, s_enc=FAKE, ld_codes=16, ld_scales=4)
    setattr(d, field, value)
    st = lib.nvfp4_quantize(FAKE, 16, 32, 32, 0, 0, 0, None, ctypes.byref(d), None)
    assert st == status


def test_rht_validation(lib):
    d = _desc(codes=FAKE, scales=FAKE, amax=FAKE, s_enc=FAKE, ld_codes=16, ld_scales=4)
    assert lib.nvfp4_rht_quantize(FAKE, 24, 16, 16, 1, 0, 0, None, ctypes.byref(d), None) == -2
    assert lib.nvfp4_rht_quantize(FAKE, 32, 12, 16, 1, 0, 0, None, ctypes.byref(d), None) == -2
    assert lib.nvfp4_rht_quantize(FAKE, 32, 16, 16, 1, 3, 0, None, ctypes.byref(d), None) == -4
    d.ld_codes = 0
    assert lib.nvfp4_rht_quantize(FAKE, 32, 16, 16, 1, 0, 0, None, ctypes.byref(d), None) == -2


@pytest.mark.parametrize("case,status", [
    # (tokens, channels, ld_x, rounding, amax, amax_rht, same descriptor, out_rht.ld_codes)
    ((32, 24, 32, 0, None, None, False, 16), -2),    # channels not a multiple of 16
    ((24, 32, 32, 0, None, None, False, 16), -2),    # tokens not a multiple of 16
    ((32, 32, 32, 2, None, None, False, 16), -4),    # unknown rounding
    ((32, 32, 32, 0, FAKE, None, False, 16), -1),    # only one of the two maxima
    ((32, 32, 32, 0, None, FAKE, False, 16), -1),
    ((32, 32, 32, 0, FAKE + 2, FAKE, False, 16), -3),  # misaligned amax
    ((32, 32, 16, 0, None, None, False, 16), -2),    # ld_x < channels
    ((32, 32, 36, 0, None, None, False, 16), -3),    # ld_x not a multiple of 8
    ((32, 32, 32, 0, None, None, True, 16), -4),     # one descriptor for both results
    ((32, 32, 32, 0, None, None, False, 0), -2),     # transposed result's rows too short
])
def test_dual_validation(lib, case, status):
    tokens, channels, ld, rnd, am, amr, same, ldr = case
    d = _desc(codes=FAKE, scales=FAKE, amax=FAKE, s_enc=FAKE, ld_codes=16, ld_scales=4)
    dr = _desc(codes=FAKE, scales=FAKE, amax=FAKE, s_enc=FAKE, ld_codes=ldr, ld_scales=4)
    st = lib.nvfp4_quantize_dual(FAKE, tokens, channels, ld, 1, rnd, 0, 0, am, amr,
                                 ctypes.byref(d), ctypes.byref(d if same else dr), None)
    assert st == status
    d.codes_t = FAKE  # no transposed copies on either result
    assert lib.nvfp4_quantize_dual(FAKE, 32, 32, 32, 1, 0, 0, 0, None, None, ctypes.byref(d),
                                   ctypes.byref(dr), None) == -4


@pytest.mark.parametrize("args,status", [
    # x, rows, cols, ld_x, mode, rounding
    ((FAKE, 32, 48, 48, 0, 0), -2),         # rows mode: cols not whole blocks of 32
    ((FAKE, 48, 32, 32, 1, 0), -2),         # transposed: rows not whole blocks of 32
    ((FAKE, 32, 12, 16, 2, 0), -2),         # transposed: cols not a multiple of 8
    ((FAKE, 32, 32, 32, 3, 0), -4),         # unknown mode
    ((FAKE, 32, 32, 32, 0, 2), -4),         # unknown rounding
    ((None, 32, 32, 32, 0, 0), -1),         # null input
    ((FAKE + 8, 32, 32, 32, 0, 0), -3),     # misaligned input
    ((FAKE, 32, 32, 16, 0, 0), -2),         # ld_x < cols
])
def test_mx_quantize_validation(lib, args, status):
    x, rows, cols, ld, mode, rnd = args
    d = _desc(codes=FAKE, scales=FAKE, ld_codes=16, ld_scales=4)
    assert lib.nvfp4_mx_quantize(x, rows, cols, ld, mode, 0, rnd, 0, ctypes.byref(d), None) == status


def test_mx_out_and_gemm_validation(lib):
    def mx(rows, cols, **kw):
        d = _desc(codes=FAKE, scales=FAKE, ld_codes=32, ld_scales=4, rows=rows, cols=cols, block=2)
        for k, v in kw.items():
            setattr(d, k, v)
        return d
    q = lambda d: lib.nvfp4_mx_quantize(FAKE, 32, 64, 64, 0, 0, 0, 0, ctypes.byref(d), None)
    assert q(mx(0, 0, codes_t=FAKE)) == -4       # no transposed copies
    assert q(mx(0, 0, ld_codes=16)) == -2        # rows of 64 codes need 32 bytes
    assert q(mx(0, 0, ld_scales=2)) == -3
    assert q(mx(0, 0, scales=None)) == -1
    g = lambda a, b, c=FAKE, ldc=64, dt=1: lib.nvfp4_mx_gemm(ctypes.byref(a), ctypes.byref(b), c,
                                                             ldc, dt, None)
    assert g(mx(16, 64), mx(8, 64), dt=5) == -4
    assert g(mx(16, 64), mx(8, 64, block=0)) == -5   # an NVFP4 operand
    assert g(mx(16, 64), mx(8, 32)) == -5            # K mismatch
    assert g(mx(16, 48), mx(8, 48)) == -2            # K not whole blocks
    assert g(mx(16, 64), mx(8, 64), c=None) == -1
    assert g(mx(16, 64), mx(8, 64), ldc=4) == -2     # ldc < N
    assert g(mx(16, 64), mx(8, 64), c=FAKE + 8) == -3
    assert g(mx(1 << 27, 64), mx(8, 64)) == -2      # codes span 4 GiB: beyond 32-bit offsets


def test_rht_sized_validation(lib):
    d = _desc(codes=FAKE, scales=FAKE, amax=FAKE, s_enc=FAKE, ld_codes=32, ld_scales=4)
    q = lambda tokens, channels, size, rnd=0: lib.nvfp4_rht_quantize_sized(
        FAKE, tokens, channels, 16, size, 0, rnd, 0, None, ctypes.byref(d), None)
    assert q(64, 16, 8) == -4            # size 8: normalisation not a power of two
    assert q(64, 16, 32) == -4
    assert q(48, 16, 64) == -2           # tokens not whole 64-token chunks
    assert q(24, 16, 4) == -2            # tokens not a multiple of 16
    assert q(64, 12, 4) == -2            # channels not a multiple of 8
    assert q(64, 16, 4, rnd=3) == -4
    assert lib.nvfp4_rht_signs64(7) & 0xFFFF == lib.nvfp4_rht_sign_mask(7)


@pytest.mark.parametrize("fn", ["nvfp4_gemm", "nvfp4_gemm_fp8blk"])
def test_gemm_validation(lib, fn):
    gemm = getattr(lib, fn)

    def op(rows, cols, block=0, **kw):
        base = dict(codes=FAKE, scales=FAKE, amax=FAKE, s_enc=FAKE, rows=rows, cols=cols,
                    ld_codes=max(16, ((cols + 31) // 32) * 16), ld_scales=max(4, cols // 16),
                    block=block)
        base.update(kw)
        return _desc(**base)

    a, w = op(32, 64), op(48, 64, 1)
    assert gemm(7, ctypes.byref(a), ctypes.byref(w), FAKE, 64, 0, None) == -4
    assert gemm(0, ctypes.byref(a), ctypes.byref(w), FAKE, 64, 3, None) == -4
    assert gemm(0, ctypes.byref(a), ctypes.byref(op(48, 32, 1)), FAKE, 64, 0, None) == -5
    assert gemm(0, ctypes.byref(w), ctypes.byref(a), FAKE, 64, 0, None) == -5
    assert gemm(1, ctypes.byref(op(32, 48)), ctypes.byref(w), FAKE, 64, 0, None) == -1
    assert gemm(2, ctypes.byref(a), ctypes.byref(w), FAKE, 64, 0, None) == -5
    assert gemm(0, ctypes.byref(a), ctypes.byref(w), FAKE + 2, 64, 0, None) == -3
    assert gemm(0, ctypes.byref(a), ctypes.byref(w), FAKE, 66, 0, None) == -3
    assert gemm(0, ctypes.byref(a), ctypes.byref(w), FAKE, 16, 0, None) == -2
    assert gemm(0, ctypes.byref(a), ctypes.byref(op(40, 64, 1)), FAKE, 64, 0, None) == -2
    # an operand's codes or scales spanning more than 4 GiB (32-bit offsets in the kernels)
    assert gemm(0, ctypes.byref(op((1 << 27) + 16, 64)), ctypes.byref(w), FAKE, 64, 0, None) == -2
    assert gemm(0, ctypes.byref(a), ctypes.byref(op(48, 64, 1, ld_scales=1 << 31)), FAKE, 64, 0,
                None) == -2


def test_gemm_amax_validation(lib):
    def op(rows, cols, block=0, **kw):
        base = dict(codes=FAKE, scales=FAKE, amax=FAKE, s_enc=FAKE, rows=rows, cols=cols,
                    ld_codes=max(16, ((cols + 31) // 32) * 16), ld_scales=max(4, cols // 16),
                    block=block)
        base.update(kw)
        return _desc(**base)

    g = lib.nvfp4_gemm_amax
    a, w, a40 = op(32, 64), op(48, 64, 1), op(40, 64)
    ra, rw = ctypes.byref(a), ctypes.byref(w)
    assert g(2, ra, ctypes.byref(op(48, 64)), FAKE, 64, 1, FAKE, FAKE, None) == -4  # wgrad
    assert g(7, ra, rw, FAKE, 64, 1, FAKE, FAKE, None) == -4
    assert g(0, ra, rw, FAKE, 64, 1, None, FAKE, None) == -1          # amax_out required
    assert g(0, ra, rw, None, 64, 1, FAKE, FAKE, None) == -1
    assert g(0, ra, rw, FAKE + 2, 64, 1, FAKE, FAKE, None) == -3
    assert g(0, ra, rw, FAKE, 64, 1, FAKE + 2, FAKE, None) == -3
    assert g(0, ra, rw, FAKE, 64, 1, FAKE, FAKE + 1, None) == -3
    assert g(0, ra, rw, FAKE, 16, 1, FAKE, FAKE, None) == -2          # ldc < N
    assert g(0, ctypes.byref(a40), rw, FAKE, 64, 1, FAKE, FAKE, None) == -2  # 40 rows with RHT
    assert g(0, rw, ra, FAKE, 64, 1, FAKE, FAKE, None) == -5
    assert g(1, ctypes.byref(op(32, 48)), rw, FAKE, 64, 1, FAKE, FAKE, None) == -1  # no W^T


def test_amax_validation(lib):
    out = FAKE
    assert lib.nvfp4_amax(FAKE, 16, 12, 16, 1, out, out, None) == -2      # cols % 8
    assert lib.nvfp4_amax(FAKE, 24, 16, 16, 1, out, out, None) == -2      # RHT rows % 16
    assert lib.nvfp4_amax(FAKE, 16, 16, 16, 1, None, out, None) == -1     # no amax output
    assert lib.nvfp4_amax(None, 16, 16, 16, 1, out, None, None) == -1     # null input
    assert lib.nvfp4_amax(FAKE + 8, 16, 16, 16, 1, out, None, None) == -3  # misaligned input
    assert lib.nvfp4_amax(FAKE, 16, 16, 8, 1, out, None, None) == -2      # ld < cols


def test_bf16_gemm_validation(lib):
    f = lib.nvfp4_bf16_gemm
    # pass, a, lda, b, ldb, M, N, K, c, ldc, dtype
    assert f(3, FAKE, 64, FAKE, 64, 16, 16, 64, FAKE, 64, 0, None) == -4      # unknown pass
    assert f(0, FAKE, 64, FAKE, 64, 16, 16, 64, FAKE, 64, 2, None) == -4      # unknown dtype
    assert f(0, FAKE, 64, FAKE, 64, 12, 16, 64, FAKE, 64, 0, None) == -2      # M % 8
    assert f(0, FAKE, 64, FAKE, 64, 16, 16, 60, FAKE, 64, 0, None) == -2      # K % 8
    assert f(0, FAKE, 64, FAKE, 64, -8, 16, 64, FAKE, 64, 0, None) == -2      # negative
    assert f(0, None, 64, FAKE, 64, 16, 16, 64, FAKE, 64, 0, None) == -1      # null a
    assert f(0, FAKE, 64, FAKE, 64, 16, 16, 64, None, 64, 0, None) == -1      # null c
    assert f(0, FAKE + 8, 64, FAKE, 64, 16, 16, 64, FAKE, 64, 0, None) == -3  # misaligned a
    assert f(0, FAKE, 60, FAKE, 64, 16, 16, 56, FAKE, 64, 0, None) == -3      # lda % 8
    assert f(0, FAKE, 64, FAKE, 64, 16, 16, 64, FAKE + 8, 64, 1, None) == -3  # fp32 c alignment
    assert f(0, FAKE, 56, FAKE, 64, 16, 16, 64, FAKE, 64, 0, None) == -2      # lda < K
    assert f(1, FAKE, 8, FAKE, 64, 16, 16, 64, FAKE, 64, 0, None) == -2       # dgrad: lda < N
    assert f(2, FAKE, 16, FAKE, 64, 16, 16, 64, FAKE, 8, 0, None) == -2       # wgrad: ldc < K


def test_mfma_sustain_validation(lib):
    f = lib.nvfp4_mfma_sustain
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    # blocks, iters, operands, out
    assert f(4, 8, 0, None, None) == -1             # null out
    assert f(0, 8, 0, FAKE, None) == -2             # no workgroup
    assert f(4, 0, 0, FAKE, None) == -2             # no round
    assert f((1 << 20) + 1, 8, 0, FAKE, None) == -2  # too many workgroups
    assert f(4, (1 << 20) + 1, 0, FAKE, None) == -2  # too many rounds
    assert f(4, 8, 3, FAKE, None) == -4             # unknown operand kind
    assert f(4, 8, -1, FAKE, None) == -4
    assert f(4, 8, 1, FAKE + 2, None) == -3         # misaligned out


def test_layout_validation(lib):
    """The code layout field: unknown values are refused, interleaved code
    rows must be whole 32-byte pieces, and the MXFP4 entry points take the
    row-major layout only."""
    base = dict(codes=FAKE, scales=FAKE, amax=FAKE, s_enc=FAKE, ld_codes=16, ld_scales=4)
    q = lambda d: lib.nvfp4_quantize(FAKE, 16, 32, 32, 0, 0, 0, None, ctypes.byref(d), None)
    assert q(_desc(**base, layout=2)) == -4
    assert q(_desc(**base, layout=-1)) == -4
    assert q(_desc(**base, layout=1)) == -3          # 16-byte code rows
    w = _desc(**dict(base, ld_codes=32, codes_t=FAKE, scales_t=FAKE, ld_codes_t=48, ld_scales_t=4,
                     layout=1))
    assert lib.nvfp4_quantize(FAKE, 32, 64, 64, 1, 0, 0, None, ctypes.byref(w), None) == -3
    r = _desc(**base, layout=1)  # channels x tokens = 16 x 32: 16-byte rows
    assert lib.nvfp4_rht_quantize(FAKE, 32, 16, 16, 1, 0, 0, None, ctypes.byref(r), None) == -3
    assert lib.nvfp4_rht_quantize_sized(FAKE, 32, 16, 16, 16, 0, 0, 0, None, ctypes.byref(r),
                                        None) == -3
    assert lib.nvfp4_quantize_rht_rows(FAKE, 16, 32, 32, 0, 1, 0, 0, None, ctypes.byref(r),
                                       None) == -3
    d = _desc(**dict(base, ld_codes=32))
    assert lib.nvfp4_quantize_dual(FAKE, 32, 32, 32, 1, 0, 0, 0, None, None, ctypes.byref(d),
                                   ctypes.byref(_desc(**base, layout=1)), None) == -3

    def op(rows, cols, block=0, **kw):
        b = dict(codes=FAKE, scales=FAKE, amax=FAKE, s_enc=FAKE, rows=rows, cols=cols,
                 ld_codes=max(16, ((cols + 31) // 32) * 16), ld_scales=max(4, cols // 16),
                 block=block)
        b.update(kw)
        return _desc(**b)
    for fn in ("nvfp4_gemm", "nvfp4_gemm_fp8blk"):
        g = getattr(lib, fn)
        assert g(0, ctypes.byref(op(32, 32, layout=1)), ctypes.byref(op(48, 32, 1)), FAKE, 64, 0,
                 None) == -3
        assert g(0, ctypes.byref(op(32, 64, layout=5)), ctypes.byref(op(48, 64, 1)), FAKE, 64, 0,
                 None) == -4
        wt = op(48, 64, 1, layout=1, ld_codes=32, codes_t=FAKE, scales_t=FAKE, ld_codes_t=48,
                ld_scales_t=4)  # dgrad reads the transposed copy: 48-byte rows
        assert g(1, ctypes.byref(op(32, 48)), ctypes.byref(wt), FAKE, 64, 0, None) == -3

    mx = lambda rows, cols, **kw: _desc(**dict(dict(codes=FAKE, scales=FAKE, ld_codes=32,
                                                    ld_scales=4, rows=rows, cols=cols, block=2),
                                               **kw))
    assert lib.nvfp4_mx_quantize(FAKE, 32, 64, 64, 0, 0, 0, 0, ctypes.byref(mx(0, 0, layout=1)),
                                 None) == -4
    assert lib.nvfp4_mx_gemm(ctypes.byref(mx(16, 64, layout=1)), ctypes.byref(mx(8, 64)), FAKE,
                             64, 1, None) == -4
