"""The interleaved code layout (nvfp4_tensor.layout = 1) against its
definition in include/nvfp4.h: byte j of code row r lies at flat offset
(r // 4) * 4 * ld + (j // 32) * 128 + (r % 4) * 32 + j % 32.  CPU only: the
binding's host conversions (used to read interleaved codes back) are checked
byte by byte against that formula, evaluated here with plain loops."""
import numpy as np
import pytest

import quantize_precision_gemm_amd as q


def _by_formula(codes):
    rows, ld = codes.shape
    out = np.zeros(((rows + 3) // 4 * 4) * ld, dtype=np.uint8)
    for r in range(rows):
        for j in range(ld):
            out[(r // 4) * 4 * ld + (j // 32) * 128 + (r % 4) * 32 + j % 32] = codes[r, j]
    return out


@pytest.mark.parametrize("rows,ld", [(1, 32), (3, 32), (4, 64), (5, 96), (13, 160), (16, 32)])
def test_interleave_matches_the_definition(rows, ld):
    rng = np.random.default_rng(rows * 1000 + ld)
    codes = rng.integers(0, 256, size=(rows, ld), dtype=np.uint8)
    il = q.interleave_codes(codes)
    assert il.shape == ((rows + 3) // 4 * 4, ld)
    np.testing.assert_array_equal(il.reshape(-1), _by_formula(codes))
    np.testing.assert_array_equal(q.deinterleave_codes(il, rows), codes)


def test_a_k_step_of_four_rows_is_one_line():
    # 8 rows x 128 bytes: K step s (bytes 32 s .. 32 s + 31) of rows 4 g .. 4 g + 3
    # occupies bytes [128 (4 g + s), 128 (4 g + s) + 128) of the buffer, rows in order
    rows, ld = 8, 128
    codes = np.arange(rows * ld, dtype=np.int64).reshape(rows, ld) % 251
    codes = codes.astype(np.uint8)
    flat = q.interleave_codes(codes).reshape(-1)
    for g in range(rows // 4):
        for s in range(ld // 32):
            line = flat[128 * (4 * g + s): 128 * (4 * g + s) + 128]
            want = np.concatenate([codes[4 * g + i, 32 * s: 32 * s + 32] for i in range(4)])
            np.testing.assert_array_equal(line, want)


def test_interleave_rejects_partial_pieces():
    with pytest.raises(ValueError):
        q.interleave_codes(np.zeros((4, 16), dtype=np.uint8))
    with pytest.raises(ValueError):
        q.deinterleave_codes(np.zeros((6, 32), dtype=np.uint8), 5)


def test_buffer_shapes():
    assert q._code_buf_shape(13, 80, q.LAYOUT_ROW_MAJOR) == (13, 48)
    assert q._code_buf_shape(13, 80, q.LAYOUT_INTERLEAVED) == (16, 64)
    assert q._code_buf_shape(16, 64, q.LAYOUT_INTERLEAVED) == (16, 32)
